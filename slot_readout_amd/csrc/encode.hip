// Encoder-mode forward over the prompts: the layout of the causal attention.
//
// thakicloud, "What is DiffusionGemma": the encoder mode runs the model over
// the prompt (left-to-right attention) and fills the KV cache that the
// decoder-mode denoise step reads.  The block's q, k, v projections, its
// attention and its output projection are the denoise step's own kernels; the
// prompts are cut into chunks of C tokens, each run as one "canvas" whose
// prompt part is the sequence's tokens before the chunk and whose canvas part
// is causal (AttnArgs::chunks).  The kernels here build the chunk table and
// the chunks' token ids, and copy the chunks' rows back to token order.
#include "common.h"
#include "kernels.h"

namespace dg {

// Chunk cb = b * J + jj holds chunk j = J - 1 - jj of sequence b (the longest
// chunks first, so the grid's last workgroups are the short ones).  Offsets are
// clamped as the decoder's attention clamps them (DG_FLAG_BAD_SEQLENS).
__global__ __launch_bounds__(256) void encode_plan_kernel(EncodeArgs a) {
  const int cb = blockIdx.x;
  const int b = cb / a.J, j = a.J - 1 - cb % a.J;
  int64_t p0 = a.cu[b], p1 = a.cu[b + 1];
  bool bad = false;
  if (p0 < 0) { p0 = 0; bad = true; }
  if (p1 > a.total_len) { p1 = a.total_len; bad = true; }
  if (p1 < p0) { p1 = p0; bad = true; }
  if (p1 - p0 > a.max_len) { p1 = p0 + a.max_len; bad = true; }
  if (bad && a.flags && threadIdx.x == 0 && j == 0) atomicOr(a.flags, DG_FLAG_BAD_SEQLENS);
  const int64_t start = (int64_t)j * a.C;
  const int64_t left = p1 - p0 - start;
  const int clen = left <= 0 ? 0 : (left < a.C ? (int)left : a.C);
  if (threadIdx.x == 0) {
    a.chunks[cb] = make_int4((int)p0, clen ? (int)start : 0, clen, 0);
    a.active[cb] = clen > 0;
  }
  for (int i = threadIdx.x; i < a.C; i += 256)
    a.ids_pad[(int64_t)cb * a.C + i] = i < clen ? a.prompt_ids[p0 + start + i] : 0;
}

// row i < z of chunk cb -> token row x + y + i: hidden (d values) and, when
// asked, the attention output (nq values), copied as 16-byte pieces
__global__ __launch_bounds__(256) void encode_scatter_kernel(EncodeArgs a) {
  const int cb = blockIdx.y;
  const int4 c = a.chunks[cb];
  const int64_t h16 = a.h_row_bytes / 16, o16 = a.o_row_bytes / 16;
  const int64_t per = h16 + (a.attn_out ? o16 : 0);
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < (int64_t)c.z * per;
       e += (int64_t)gridDim.x * 256) {
    const int64_t i = e / per, r = e % per;
    const int64_t src = (int64_t)cb * a.C + i, dst = (int64_t)c.x + c.y + i;
    if (r < h16)
      reinterpret_cast<uint4 *>(a.hidden_out)[dst * h16 + r] =
          reinterpret_cast<const uint4 *>(a.h_pad)[src * h16 + r];
    else
      reinterpret_cast<uint4 *>(a.attn_out)[dst * o16 + (r - h16)] =
          reinterpret_cast<const uint4 *>(a.o_pad)[src * o16 + (r - h16)];
  }
}

hipError_t launch_encode_plan(const EncodeArgs &a, hipStream_t st) {
  if ((int64_t)a.B * a.J <= 0) return hipSuccess;
  hipLaunchKernelGGL(encode_plan_kernel, dim3((unsigned)((int64_t)a.B * a.J)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_encode_scatter(const EncodeArgs &a, hipStream_t st) {
  const int64_t nc = (int64_t)a.B * a.J;
  if (nc <= 0) return hipSuccess;
  if (a.h_row_bytes % 16 || a.o_row_bytes % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(encode_scatter_kernel, dim3(16, (unsigned)nc), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dg
