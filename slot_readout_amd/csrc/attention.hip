// Decoder-mode attention for gfx950: every canvas query attends to all cached
// prompt keys of its sequence plus the canvas keys within +-W of it
// (bidirectional, no causal mask).
//
// Work split: one workgroup = (canvas, query head, tile of NQ consecutive
// canvas positions, split).  A query tile's keys -- every prompt key, then the
// canvas keys its window can reach -- are cut into equal splits (split-KV).
// Queries may instead be gathered (a few positions per canvas, e.g. the slots
// a read needs): a tile then holds NQ of them and every canvas key is a
// candidate, masked per query.
// With one split the workgroup writes the normalised output; otherwise it
// writes (m, l, unnormalised O) partials that a second kernel merges in a
// fixed order.
//
// Inside a workgroup the 4 waves each own QB x 16 query columns.  Scores are
// computed transposed, S^T = K Q^T, so that a lane holds one query column and
// the running max of that query stays in the lane (plus one exchange across
// the four 16-lane groups).  P^T then feeds O^T += V^T P^T directly from
// registers.  For bf16, K and V are both staged row-major in LDS from
// coalesced loads; the V^T fragments come from transposing LDS reads
// (ds_read_b64_tr_b16).  V carries an extra column of ones, so the same MFMA
// also accumulates the softmax denominator sum_key p (for bf16 that block of
// V^T is a constant fragment held in registers, not read from LDS).
// The waves raise their priority while they issue MFMAs: a wave that is ready
// to issue them goes ahead of the softmax work of the other waves on its SIMD,
// so the matrix cores idle less (long read at head_dim 64: 60 -> 55 us).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dg {

template <typename T, int HD> struct AttnShape;
// NW: waves per workgroup; QB: 16-query column blocks per wave; NK: keys per
// LDS block; PF: K/V blocks whose global loads are in flight ahead of the one
// being computed (a ring of register stages; 1 = load the next block only
// after the current one)
template <> struct AttnShape<bf16, 64> { static constexpr int NW = 8, QB = 1, NK = 64, PF = 2; };
template <> struct AttnShape<float, 64> { static constexpr int NW = 4, QB = 2, NK = 64, PF = 2; };
template <> struct AttnShape<bf16, 512> { static constexpr int NW = 4, QB = 1, NK = 32, PF = 1; };

typedef short v4s __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16: within each 16-lane group, output lane 4a+b element j is
// element b of the 8 bytes addressed by source lane a+4j of the group
__device__ inline v4s ds_read_tr16(const void *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s *)(p));
}

// one 16-byte chunk per lane from global memory straight into LDS: lane l
// writes bytes [16 l, 16 l + 16) after dst (dst must be wave-uniform)
__device__ inline void lds_row16(const void *src, void *dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
}

__device__ inline void pin4(uint4 &v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

constexpr float kLazy = 8.f;
// owners in the key table of a patched tile
constexpr int kKeyShared = 0xFE, kKeyNone = 0xFF;

// Split partials of O are kept in the storage type: fp32, or bf16 whose
// rounding (2^-9 relative) matches that of the final bf16 output.
template <typename T> __device__ inline void store4v(T *p, f32x4 v);
template <> __device__ inline void store4v<float>(float *p, f32x4 v) {
  *reinterpret_cast<f32x4 *>(p) = v;
}
template <> __device__ inline void store4v<bf16>(bf16 *p, f32x4 v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 b = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *reinterpret_cast<bf16x4 *>(p) = b;
}
template <typename T> __device__ inline float4 load4v(const T *p);
template <> __device__ inline float4 load4v<float>(const float *p) {
  return *reinterpret_cast<const float4 *>(p);
}
template <> __device__ inline float4 load4v<bf16>(const bf16 *p) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
  return make_float4((float)b[0], (float)b[1], (float)b[2], (float)b[3]);
}

// Keys of the query tile starting at query i0 of canvas cb, in the order the
// splits cut them: every prompt key of the canvas's sequence (rows
// [p0, p0 + plen) of the cache, offsets clamped against corrupt cu_seqlens, in
// which case true is returned), then the canvas keys [lo, hi) that the tile's
// +-W window can reach (every canvas key for gathered queries).
// With ncp canvases packed in the tile (gathered queries of canvases that
// share a prompt), the canvas keys are those of the ncp canvases, one after
// the other ([0, ncp * C)).
// Patched draws (a.kpatch, gathered queries): the tile's canvases share their
// base canvas and their query positions, so the canvas keys are *na rows of
// the base canvas -- the listed union of the windows of its queries
// (a.win_cnt), else every position of [*alo, *alo + *na) from the lowest window
// start to the highest window end -- then the ncp * qn slot rows of the tile's
// canvases in kpatch ([0, *na + ncp * qn)).
// Encoder-mode chunks (a.chunks): the keys of the sequence before the chunk,
// then the chunk's own keys up to the tile's last query (none for a tile past
// the chunk's end).
__device__ inline bool tile_keys(const AttnArgs &a, int cb, int i0, int nq, int64_t *p0o,
                                 int64_t *plen, int *lo, int *hi, int ncp = 1, int *alo = nullptr,
                                 int *na = nullptr) {
  if (a.chunks) {
    const int4 c = a.chunks[cb];
    const bool past = i0 >= c.z;
    *p0o = c.x;
    *plen = past ? 0 : c.y;
    *lo = 0;
    *hi = past ? 0 : (i0 + nq < c.z ? i0 + nq : c.z);
    return false;
  }
  const int pb = cb / a.canvas_per_prompt;
  int64_t p0 = a.cu[pb], p1 = a.cu[pb + 1];
  bool bad = false;
  if (p0 < 0) { p0 = 0; bad = true; }
  if (p1 > a.total_len) { p1 = a.total_len; bad = true; }
  if (p1 < p0) { p1 = p0; bad = true; }
  if (p1 - p0 > a.max_len) { p1 = p0 + a.max_len; bad = true; }
  *p0o = p0;
  *plen = p1 - p0;
  if (a.qpos && a.kpatch && a.win_cnt) {
    const int n = a.win_cnt[cb / a.canvas_per_prompt];
    if (alo) *alo = 0;
    if (na) *na = n;
    *lo = 0;
    *hi = n + ncp * a.qn;
  } else if (a.qpos && a.kpatch) {
    int mn = a.C, mx = -1;
    for (int sl = 0; sl < a.qn; ++sl) {
      const int p = a.qpos[(int64_t)cb * a.qn + sl];
      if (p >= 0 && p < a.C) {
        mn = p < mn ? p : mn;
        mx = p > mx ? p : mx;
      }
    }
    // (the host clamps W to C - 1, so mx + W + 1 does not overflow)
    const int l0 = mx < 0 ? 0 : (mn - a.W > 0 ? mn - a.W : 0);
    const int l1 = mx < 0 ? 0 : (mx + a.W + 1 < a.C ? mx + a.W + 1 : a.C);
    if (alo) *alo = l0;
    if (na) *na = l1 - l0;
    *lo = 0;
    *hi = (l1 - l0) + ncp * a.qn;
  } else if (a.qpos) {
    *lo = 0;
    *hi = a.C * ncp;
  } else {
    *lo = i0 - a.W > 0 ? i0 - a.W : 0;
    *hi = i0 + nq + a.W < a.C ? i0 + nq + a.W : a.C;   // exclusive
  }
  return bad;
}

// PREC (bf16 only): the probabilities enter the PV product as two bf16 terms,
// p = hi + lo with hi = bf16(p) and lo = bf16(p - hi) (one more MFMA per V
// fragment), and O, its split partials and the output are fp32.  The result
// then carries the rounding of the stored q, k, v only, not that of p and o.
// PATCH (a read's draws, a.kpatch set): canvas cb's canvas keys are those of
// its base canvas cb / canvas_per_prompt, except at the slot positions of the
// draws (canvases with cb % canvas_per_prompt >= patch_from), whose keys and
// values are the slot rows cb * qn + s of kpatch / vpatch: the draws differ
// from their base canvas only there, so no draw canvas's k, v are stored.
// HK > 1 (patched tiles, bf16, head_dim 64): the workgroup serves all HK kv
// heads of its canvases: K/V rows are staged whole (HK heads side by side) and
// each wave takes the columns of one kv head (NQ / HK columns per head), so the
// gathered queries of every head compute on one staging of the keys.
template <typename T, int HD, bool PREC = false, bool PATCH = false, int HK = 1>
__global__ __launch_bounds__((64 * AttnShape<T, HD>::NW), (HK > 1 ? 2 : (HD == 64 && sizeof(T) == 2 ? 4 : 1))) void attn_kernel(AttnArgs a) {
  using MF = Mfma<T>;
  using frag = typename MF::frag;
  constexpr int QB = AttnShape<T, HD>::QB;
  constexpr int NK = AttnShape<T, HD>::NK;
  constexpr int PF = AttnShape<T, HD>::PF;
  constexpr int NW = AttnShape<T, HD>::NW;
  constexpr int NT = 64 * NW;
  constexpr int NQ = NW * QB * 16;
  constexpr int VEC = 16 / sizeof(T);
  constexpr bool TR = sizeof(T) == 2;
  static_assert(!PREC || TR, "split probabilities: bf16 storage");
  // slot index at each canvas position of the tile's canvases (-1: none), and
  // the table of the tile's canvas keys (see tile_keys): position | owner << 16
  // | slot-position flag << 24, owner kKeyShared for a base row (seen by every
  // canvas of the tile, except by a draw at one of its slot positions), a canvas
  // j of the tile for its slot row, or kKeyNone
  __shared__ short smap[PATCH ? DG_MAX_CANVAS : 1];
  __shared__ int kinfo[PATCH ? 2 * DG_MAX_CANVAS : 1];
  // output / partial type
  using TO = typename std::conditional<PREC, float, T>::type;
  // bf16 rows of K and V are HD + 16 elements apart: with that stride both the
  // 16-byte K fragment reads and the transposing V reads are free of LDS bank
  // conflicts (measured on gfx950; a 16-byte pad leaves 2-way conflicts)
  static_assert(HK == 1 || (PATCH && TR && HD == 64), "packed kv heads: patched bf16 tiles at head_dim 64");
  constexpr int RW = HK * HD;                   // elements of a staged key row
  constexpr int KP = TR ? RW + 16 : RW + VEC;
  constexpr int VP = NK + VEC;
  constexpr int KS = HD / MF::KI;
  constexpr int CPK = RW / VEC;                 // 16-byte chunks per key row
  constexpr int CH = NK * CPK / NT;             // chunks of K (and of V) per thread per block
  static_assert(NK * CPK % NT == 0, "block/thread mismatch");
  // K and V tiles are double-buffered: block b lives in buffer b % 2, so the
  // next block can be staged while the current one is read, one barrier apart
  // (each buffer its own array: the compiler then sees that reads of one buffer
  // do not depend on direct-to-LDS loads into the other)
  __shared__ __attribute__((aligned(16))) T Ks0[NK * KP], Ks1[NK * KP];
  auto Ks = [&](int bf) -> T * { return bf ? Ks1 : Ks0; };
  // V plus one extra 16-wide block whose first element is 1: the PV MFMA then
  // also yields sum_key p (the softmax denominator).  bf16: V row-major [NK][VKP]
  // read through transposing LDS reads (the extra block is a register constant;
  // its 16 columns in LDS only pad the rows); fp32: V^T [RB*16][VP] staged
  // element-wise, with the extra block.
  constexpr int RB = HD / 16 + 1;
  constexpr int VKP = RW + 16;
  constexpr int VSZ = TR ? NK * VKP : RB * 16 * VP;
  __shared__ __attribute__((aligned(16))) T Vt0[VSZ], Vt1[VSZ];
  auto Vt = [&](int bf) -> T * { return bf ? Vt1 : Vt0; };

  // group = (canvas, kv head, split); its tiles (the query heads sharing the
  // kv head x the query tiles) read the same K/V blocks and run on one XCD.
  // With ncp > 1 a tile holds the gathered queries of ncp consecutive canvases
  // that share a prompt (a read's draws): the prompt's K/V blocks are staged
  // once for all of them.
  const int QN = a.qpos ? a.qn : a.C;   // queries per canvas
  const int nqt = (QN + NQ - 1) / NQ;
  const int ncp = a.cpack > 1 ? a.cpack : 1;
  int grpi, tile;
  const int hkg = HK > 1 ? 1 : a.Hkv;   // kv-head groups per canvas group
  if (!xcd_group_tile(a.nc / ncp * hkg * a.nsplit, (HK > 1 || a.packed) ? 1 : (a.Hq / a.Hkv) * nqt, &grpi, &tile))
    return;
  const int s = grpi % a.nsplit;
  const int cb = grpi / a.nsplit / hkg * ncp;   // the tile's first canvas
  // packed: h is the kv group's first query head and every column names its own
  // (HK > 1: h = 0 and the columns name their heads)
  const int h = HK > 1 ? 0 : (grpi / a.nsplit % a.Hkv) * (a.Hq / a.Hkv) + (a.packed ? 0 : tile / nqt);
  const int qt = a.packed ? 0 : tile % nqt;
  if (a.active && ncp == 1 && !a.active[cb]) return;
  const int G = a.Hq / a.Hkv, g = h / G;
  const int C = a.C, W = a.chunks ? a.C - 1 : a.W;
  const int Wup = a.chunks ? 0 : W;   // reach of the window after the query
  const int i0 = qt * NQ;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;

  int64_t p0, plen;
  int lo, hi, alo = 0, na = 0;
  const bool bad = tile_keys(a, cb, i0, NQ, &p0, &plen, &lo, &hi, ncp, &alo, &na);
  if (bad && a.flags && threadIdx.x == 0 && s == 0 && qt == 0 && h == 0)
    atomicOr(a.flags, DG_FLAG_BAD_SEQLENS);
  const int64_t nkeys = plen + (hi - lo);
  const int64_t vb0 = (int64_t)s * a.chunk;
  // splits past this tile's keys (shorter prompts of a ragged batch) have
  // nothing to do; the merge reads only the splits that hold keys
  if (vb0 >= nkeys && a.nsplit > 1) return;
  const int64_t vb1 = vb0 + a.chunk < nkeys ? vb0 + a.chunk : nkeys;
  const int64_t ps = p0 + (vb0 < plen ? vb0 : plen);
  const int64_t pe = p0 + (vb1 < plen ? vb1 : plen);
  const int cs0 = lo + (int)(vb0 > plen ? vb0 - plen : 0);
  const int cs1 = lo + (int)(vb1 > plen ? vb1 - plen : 0);
  const int np = pe > ps ? (int)((pe - ps + NK - 1) / NK) : 0;   // prompt blocks
  const int nc = cs1 > cs0 ? (cs1 - cs0 + NK - 1) / NK : 0;     // canvas blocks

  const int64_t kv_stride = (int64_t)a.Hkv * HD;   // elements between consecutive keys
  const int64_t q_stride = (int64_t)a.Hq * HD;
  // q rows: canvas positions, or the compact rows of gathered queries
  const T *qbase = static_cast<const T *>(a.q) + (int64_t)cb * (a.qpos ? QN : C) * q_stride +
                   (int64_t)h * HD;
  // query index, head and canvas (offset from cb) of each of the lane's
  // columns (packed: c -> canvas c / (G QN), head c / QN % G, query c % QN)
  int cq[QB], chd[QB], ccv[QB];
#pragma unroll
  for (int jb = 0; jb < QB; ++jb) {
    const int c = i0 + w * QB * 16 + jb * 16 + col;
    if constexpr (HK > 1) {
      // column c: kv head c / (NQ / HK), then the packed order within the head
      constexpr int CPH = NQ / HK;
      const int lc = c % CPH;
      const bool in = lc < ncp * G * QN;
      cq[jb] = in ? lc % QN : QN;
      chd[jb] = in ? c / CPH * G + lc / QN % G : 0;
      ccv[jb] = in ? lc / (G * QN) : 0;
    } else {
      const bool in = c < ncp * G * QN;
      cq[jb] = a.packed ? (in ? c % QN : QN) : c;
      chd[jb] = a.packed ? (in ? c / QN % G : 0) : 0;
      ccv[jb] = a.packed && in ? c / (G * QN) : 0;
    }
  }
  // offset of the wave's kv head in a staged row (HK > 1)
  static_assert(HK == 1 || (NQ / HK) % (QB * 16) == 0, "a wave's columns within one kv head");
  const int gofs = HK > 1 ? (w * QB * 16) / (NQ / HK) * HD : 0;
  const T *kp = static_cast<const T *>(a.kp) + (int64_t)g * HD;
  const T *vp = static_cast<const T *>(a.vp) + (int64_t)g * HD;
  const int64_t cbase = (int64_t)cb * (a.kv_cmul > 1 ? a.kv_cmul : 1) * C * kv_stride + (int64_t)g * HD;
  const int cpp = a.canvas_per_prompt;
  if constexpr (PATCH) {
    // the canvases of a tile are draws of one base canvas: they share its slot
    // positions; in slot order, so a later slot at the same position wins
    for (int i = threadIdx.x; i < C; i += NT) smap[i] = -1;
    __syncthreads();
    if (threadIdx.x == 0)
      for (int sl = 0; sl < QN; ++sl) {
        const int p = a.qpos[(int64_t)cb * QN + sl];
        if (p >= 0 && p < C) smap[p] = (short)sl;
      }
    __syncthreads();
    for (int kk = threadIdx.x; kk < na; kk += NT) {
      const int p = a.win_pos ? a.win_pos[(int64_t)(cb / cpp) * C + kk] : alo + kk;
      kinfo[kk] = p | (kKeyShared << 16) | (smap[p] >= 0 ? 1 << 24 : 0);
    }
    for (int kb = threadIdx.x; kb < ncp * QN; kb += NT) {
      const int j = kb / QN, sl = kb % QN;
      const int p = a.qpos[(int64_t)(cb + j) * QN + sl];
      // the slot row of a draw at its position, unless a later slot there wins
      const bool own = p >= 0 && p < C && (cb + j) % cpp >= a.patch_from && smap[p] == sl;
      kinfo[na + kb] = own ? p | (j << 16) : kKeyNone << 16;
    }
    __syncthreads();
  }
  const T *kc = static_cast<const T *>(a.k) + cbase;
  const T *vc = static_cast<const T *>(a.v) + cbase;

  // canvas position of each query column of the lane (packed canvases: in the
  // concatenation of the tile's canvases, ccv * C + position); a column past
  // the canvas (or a gathered query without a position, or of an inactive
  // canvas) loads zeros and sees no canvas key
  int qp[QB];
#pragma unroll
  for (int jb = 0; jb < QB; ++jb) {
    const int qi = cq[jb];
    int p = qi;
    if (a.qpos) p = qi < QN ? a.qpos[(int64_t)(cb + ccv[jb]) * QN + qi] : -1;
    if (ncp > 1 && a.active && !a.active[cb + ccv[jb]]) p = -1;
    if (a.chunks && p >= a.chunks[cb].z) p = -1;   // past the chunk's tokens
    qp[jb] = p >= 0 && p < C ? ccv[jb] * C + p : -(1 << 20);
  }
  // a wave none of whose columns holds a query (past the canvas end, or past
  // the few gathered queries of a read) only helps stage K and V
  bool has_q = false;
#pragma unroll
  for (int jb = 0; jb < QB; ++jb) has_q |= qp[jb] >= 0;
  const bool live = __builtin_amdgcn_readfirstlane((int)__any(has_q)) != 0;
  frag qf[QB][KS];
#pragma unroll
  for (int jb = 0; jb < QB; ++jb) {
    const int qrow = a.qpos ? ccv[jb] * QN + cq[jb] : qp[jb];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (qp[jb] >= 0)
        qf[jb][ks] = *reinterpret_cast<const frag *>(qbase + (int64_t)qrow * q_stride +
                                                      (int64_t)chd[jb] * HD + ks * MF::KI +
                                                      grp * MF::KPL);
      else
        qf[jb][ks] = frag{};
    }
  }
  // Q is complete before the K/V ring starts: otherwise the wait for the Q
  // loads inside the loop would also drain every ring load issued after them
#pragma unroll
  for (int jb = 0; jb < QB; ++jb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint32_t *u = reinterpret_cast<uint32_t *>(&qf[jb][ks]);
#pragma unroll
      for (int e = 0; e < (int)(sizeof(frag) / 4); ++e) asm volatile("" : "+v"(u[e]));
    }

  f32x4 oacc[RB][QB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int jb = 0; jb < QB; ++jb) oacc[rb][jb] = zero4();
  float mrun[QB];
#pragma unroll
  for (int jb = 0; jb < QB; ++jb) mrun[jb] = -INFINITY;
  // the block of V^T past the head: row HD is all ones, the rest zeros.  bf16:
  // lane (col, grp) of a fragment holds row HD + col, so the fragment is a
  // constant; fp32: staged once in both LDS buffers
  frag ones_frag{};
  if constexpr (TR) {
#pragma unroll
    for (int e = 0; e < MF::KPL; ++e) ones_frag[e] = from_f<T>(col == 0 ? 1.f : 0.f);
  } else {
#pragma unroll
    for (int bf = 0; bf < 2; ++bf)
      for (int i = threadIdx.x; i < 16 * VP; i += NT) Vt(bf)[HD * VP + i] = from_f<T>(i < VP ? 1.f : 0.f);
  }

  // block b: prompt blocks first, then canvas-window blocks; b >= nb names an
  // empty block (every lane loads the first canvas key, and nothing is used)
  const int nb = np + nc;
  const int64_t bstride = (int64_t)NK * kv_stride;   // elements between consecutive blocks
  const T *kp0 = kp + ps * kv_stride, *vp0 = vp + ps * kv_stride;
  const T *kc0 = kc + (int64_t)cs0 * kv_stride, *vc0 = vc + (int64_t)cs0 * kv_stride;
  const int prem = (int)(pe - ps), crem = cs1 - cs0;   // prompt / canvas keys of the split
  // Blocks are read through buffer resources whose size covers only the block's
  // valid keys: loads of rows past the end return zeros without touching memory.
  struct Blk { const T *kb, *vb; int k0; int rem; bool canvas; };
  auto desc = [&](int b) {
    Blk d;
    if (b >= nb) {
      d.k0 = 0;
      d.kb = kc;
      d.vb = vc;
      d.rem = 0;
      d.canvas = true;
    } else if (b < np) {
      d.k0 = 0;   // prompt keys are visible to every query: no position needed
      d.kb = kp0 + b * bstride;
      d.vb = vp0 + b * bstride;
      d.rem = min(prem - b * NK, NK);
      d.canvas = false;
    } else {
      const int bc = b - np;
      d.k0 = cs0 + bc * NK;
      d.kb = kc0 + bc * bstride;
      d.vb = vc0 + bc * bstride;
      d.rem = min(crem - bc * NK, NK);
      d.canvas = true;
    }
    return d;
  };
  // Per-thread chunk assignment, fixed for every block.  K chunk i: key c / CPK,
  // chunk c % CPK (lanes along a row).  bf16 V is loaded the same way; fp32 V
  // takes key c % NK, chunk c / NK (lanes along keys, so the element-wise
  // transposed stores hit neighbouring positions).
  int kkey[CH], vkey[CH], kgo[CH], vgo[CH], klo[CH], vlo[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = i * NT + threadIdx.x;
    kkey[i] = c / CPK;
    kgo[i] = kkey[i] * (int)kv_stride + (c % CPK) * VEC;
    klo[i] = kkey[i] * KP + (c % CPK) * VEC;
    if constexpr (TR) {   // V row-major, same coalesced pattern as K
      vkey[i] = kkey[i];
      vgo[i] = kgo[i];
      vlo[i] = kkey[i] * VKP + (c % CPK) * VEC;
    } else {
      vkey[i] = c % NK;
      vgo[i] = vkey[i] * (int)kv_stride + (c / NK) * VEC;
      vlo[i] = (c / NK) * VEC * VP + vkey[i];
    }
  }
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  // head_dim 512 (bf16): a key row of K or V is 1 KB, one direct-to-LDS wave
  // instruction (64 lanes x 16 bytes), so the blocks are staged straight into
  // LDS and no registers hold them
  constexpr bool DMA = TR && HD == 512 && !PATCH;
  u32x4 kr[DMA ? 1 : PF][DMA ? 1 : CH], vr[DMA ? 1 : PF][DMA ? 1 : CH];
  // PATCH: the source of row r of block d (plain loads with per-lane
  // addresses): prompt rows from the block (blk), canvas rows from the base
  // canvas (base) or the draw's slot rows (patch).  Rows past the block's keys
  // read its first row: their scores are masked and their probabilities 0.
  auto src_row = [&](const Blk &d, int r, const T *blk, const T *base, const T *patch) -> const T * {
    const int rr = r < d.rem ? r : 0;
    if (!d.canvas) return blk + (int64_t)rr * kv_stride;
    const int kk = d.k0 + rr;   // canvas key of the tile: a base row, then the slot rows
    return kk < na ? base + ((int64_t)(cb / cpp) * C + (kinfo[kk] & 0xFFFF)) * kv_stride
                   : patch + ((int64_t)cb * QN + (kk - na)) * kv_stride + (int64_t)g * HD;
  };
  auto fetch = [&](const Blk &d, u32x4 (&xk)[CH], u32x4 (&xv)[CH]) {
    if constexpr (PATCH) {
      const T *kb0 = static_cast<const T *>(a.k) + (int64_t)g * HD;
      const T *vb0 = static_cast<const T *>(a.v) + (int64_t)g * HD;
      const T *kpt = static_cast<const T *>(a.kpatch), *vpt = static_cast<const T *>(a.vpatch);
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int kcol = kgo[i] - kkey[i] * (int)kv_stride, vcol = vgo[i] - vkey[i] * (int)kv_stride;
        xk[i] = *reinterpret_cast<const u32x4 *>(src_row(d, kkey[i], d.kb, kb0, kpt) + kcol);
        xv[i] = *reinterpret_cast<const u32x4 *>(src_row(d, vkey[i], d.vb, vb0, vpt) + vcol);
      }
      return;
    }
    const int nbytes = d.rem * (int)kv_stride * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(d.kb), (short)0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(d.vb), (short)0, nbytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      xk[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, kgo[i] * (int)sizeof(T), 0, 0);
      xv[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, vgo[i] * (int)sizeof(T), 0, 0);
    }
  };
  auto stage = [&](const u32x4 (&xk)[CH], const u32x4 (&xv)[CH], int bf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      uint4 kx{xk[i].x, xk[i].y, xk[i].z, xk[i].w}, vx{xv[i].x, xv[i].y, xv[i].z, xv[i].w};
      pin4(kx);
      pin4(vx);
      *reinterpret_cast<uint4 *>(Ks(bf) + klo[i]) = kx;
      if constexpr (TR) {
        *reinterpret_cast<uint4 *>(Vt(bf) + vlo[i]) = vx;
      } else {
        Chunk<T> vch;
        vch.u = vx;
#pragma unroll
        for (int e = 0; e < VEC; ++e) Vt(bf)[vlo[i] + e * VP] = vch.v[e];
      }
    }
  };

  // Scores are in log2 units (q is pre-scaled).  Each query column keeps a
  // reference mref (its running max, 0 before the first key); the score MFMAs
  // start from -mref, so they produce s - mref directly.
  // (at hd 512 the four registers of -mref are not spared: the scores start
  // from zero and mref is subtracted afterwards, 8 values per lane)
  constexpr bool INIT_NEG = HD <= 64;
  float mref[QB];
  f32x4 negm[QB];
#pragma unroll
  for (int jb = 0; jb < QB; ++jb) {
    mref[jb] = 0.f;
    negm[jb] = zero4();
  }
  // head_dim 64 (without split probabilities): every K fragment of the block is
  // read before the first score MFMA, so the block waits for LDS once
  constexpr bool KPRE = HD == 64 && !PREC;
  // MFMA-phase priority (head_dim 64 bf16; at head_dim 512 and in fp32 the
  // priority changes cost the scheduler's freedom and registers spill)
  constexpr bool PRIO = HD == 64 && TR;
  auto compute = [&](const Blk &d, int bf) {
    f32x4 sacc[NK / 16][QB];
    auto kfrag = [&](int ks, int kb2) {
      return *reinterpret_cast<const frag *>(Ks(bf) + (kb2 * 16 + col) * KP + gofs + ks * MF::KI + grp * MF::KPL);
    };
    frag kf[KPRE ? KS : 1][KPRE ? NK / 16 : 1];
    if constexpr (KPRE) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kb2 = 0; kb2 < NK / 16; ++kb2) kf[ks][kb2] = kfrag(ks, kb2);
    }
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb2 = 0; kb2 < NK / 16; ++kb2) {
        const frag af = KPRE ? kf[KPRE ? ks : 0][KPRE ? kb2 : 0] : kfrag(ks, kb2);
#pragma unroll
        for (int jb = 0; jb < QB; ++jb)
          sacc[kb2][jb] = MF::mma(af, qf[jb][ks], ks == 0 ? (INIT_NEG ? negm[jb] : zero4()) : sacc[kb2][jb]);
      }
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    if constexpr (!INIT_NEG) {
#pragma unroll
      for (int kb2 = 0; kb2 < NK / 16; ++kb2)
#pragma unroll
        for (int jb = 0; jb < QB; ++jb) sacc[kb2][jb] -= mref[jb];
    }

    const bool full = !d.canvas && d.rem == NK;   // uniform: no key of the block is masked
#pragma unroll
    for (int jb = 0; jb < QB; ++jb) {
      if (PATCH && d.canvas) {
        // a base row is seen within the window, except by a draw at one of its
        // slot positions; a slot row only by its own canvas, within the window
        const int pq = qp[jb] - ccv[jb] * C;   // the query's position (negative: none)
        const bool cpat = (cb + ccv[jb]) % cpp >= a.patch_from;
#pragma unroll
        for (int kb2 = 0; kb2 < NK / 16; ++kb2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kl = kb2 * 16 + grp * 4 + r;
            const int info = kinfo[d.k0 + (kl < d.rem ? kl : 0)];
            const int own = (info >> 16) & 0xFF, dp = (info & 0xFFFF) - pq;
            const bool ok = kl < d.rem && qp[jb] >= 0 && dp >= -W && dp <= W &&
                            (own == kKeyShared ? !(cpat && (info >> 24)) : own == ccv[jb]);
            sacc[kb2][jb][r] = ok ? sacc[kb2][jb][r] : -INFINITY;
          }
      } else if (!full) {
        // canvas keys: visible iff |key - qp| <= W, i.e. kl in [qrel - W, qrel +
        // W], and (packed canvases) the key is of the column's own canvas
        const int qrel = qp[jb] - d.k0;
        const int cv0 = ccv[jb] * C - d.k0;   // the column's canvas: [cv0, cv0 + C)
        // (encoder-mode chunks: keys at or before the query, W = C - 1)
        const int klo_ok = d.canvas ? max(qrel - W, cv0) : -1;
        const int khi_ok = d.canvas ? min(min(qrel + Wup, cv0 + C - 1), d.rem - 1) : d.rem - 1;
        // key kl = kb2 * 16 + grp * 4 + r, compared as kb2 * 16 + r against the
        // bounds less grp * 4: the offsets are inline constants, not registers
        const int glo = klo_ok - grp * 4, ghi = khi_ok - grp * 4;
#pragma unroll
        for (int kb2 = 0; kb2 < NK / 16; ++kb2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kc = kb2 * 16 + r;
            const bool ok = kc >= glo && kc <= ghi;
            sacc[kb2][jb][r] = ok ? sacc[kb2][jb][r] : -INFINITY;
          }
      }
      float bm = -INFINITY;   // block max relative to mref
#pragma unroll
      for (int kb2 = 0; kb2 < NK / 16; ++kb2)
#pragma unroll
        for (int r = 0; r < 4; ++r) bm = fmaxf(bm, sacc[kb2][jb][r]);
      bm = group4_max(bm);
      // The reference is raised only when the block's max exceeds it by more
      // than kLazy (or on the first keys); until then the exponentials stay
      // below 2^kLazy and nothing is rescaled.  The sum of p (the ones row)
      // shares the reference, so the normalised result does not depend on it.
      const bool grow = bm > kLazy || (mrun[jb] == -INFINITY && bm != -INFINITY);
      if (__any(grow)) {
        const float delta = grow ? bm : 0.f;
        const float alpha = mrun[jb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(-delta);
#pragma unroll
        for (int kb2 = 0; kb2 < NK / 16; ++kb2)
#pragma unroll
          for (int r = 0; r < 4; ++r) sacc[kb2][jb][r] -= delta;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) oacc[rb][jb] *= alpha;
        if (grow) {
          mref[jb] += delta;
          mrun[jb] = mref[jb];
          if constexpr (INIT_NEG) negm[jb] = f32x4{-mref[jb], -mref[jb], -mref[jb], -mref[jb]};
        }
      }
      // raw v_exp_f32: every argument is <= kLazy or -inf
#pragma unroll
      for (int kb2 = 0; kb2 < NK / 16; ++kb2)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[kb2][jb][r] = __builtin_amdgcn_exp2f(sacc[kb2][jb][r]);
    }

    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
    if constexpr (MF::KPL == 8) {
#pragma unroll
      for (int t = 0; t < NK / 32; ++t)
#pragma unroll
        for (int jb = 0; jb < QB; ++jb) {
          frag pf, pl;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pf[j] = (bf16)sacc[2 * t][jb][j];
            pf[4 + j] = (bf16)sacc[2 * t + 1][jb][j];
            if constexpr (PREC) {
              pl[j] = (bf16)(sacc[2 * t][jb][j] - (float)pf[j]);
              pl[4 + j] = (bf16)(sacc[2 * t + 1][jb][j] - (float)pf[4 + j]);
            }
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            // A = V^T block: lane (col=d, grp) needs keys 32t+4grp+0..3 and
            // 32t+16+4grp+0..3 for d = rb*16 + col.  A transposing read where
            // source lane s of the group points at V[key0 + s/4][d0 + 4(s%4)]
            // returns V[key0 + 0..3][d0 + lane%16] in each lane.
            frag af = ones_frag;
            if (rb < HD / 16) {
              const T *src0 = Vt(bf) + (t * 32 + grp * 4 + (col >> 2)) * VKP + gofs + rb * 16 + 4 * (col & 3);
              const v4s lo4 = ds_read_tr16(src0);
              const v4s hi4 = ds_read_tr16(src0 + 16 * VKP);
              __builtin_memcpy(&af, &lo4, 8);
              __builtin_memcpy(reinterpret_cast<char *>(&af) + 8, &hi4, 8);
            }
            oacc[rb][jb] = MF::mma(af, pf, oacc[rb][jb]);
            if constexpr (PREC) oacc[rb][jb] = MF::mma(af, pl, oacc[rb][jb]);
          }
        }
    } else {
#pragma unroll
      for (int kb2 = 0; kb2 < NK / 16; ++kb2)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const frag af = Vt(bf)[(rb * 16 + col) * VP + kb2 * 16 + grp * 4 + r];
#pragma unroll
            for (int jb = 0; jb < QB; ++jb) oacc[rb][jb] = MF::mma(af, sacc[kb2][jb][r], oacc[rb][jb]);
          }
    }
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
  };

  // Pipeline: block b is computed from LDS buffer b % 2 while block b+1 is
  // written into the other buffer from its register slot, (b+1) % PF, which is
  // then refilled with block b+1+PF; one barrier per block separates the two.
  // The loop is unrolled by U = lcm(PF, 2) so every slot and buffer index is a
  // compile-time constant.  Inside the main loop slots are refilled
  // unconditionally (past the end, with the empty block), so the loads retire
  // in issue order and each stage waits only for its own slot.
  constexpr int U = PF % 2 == 0 ? PF : 2 * PF;
  if constexpr (DMA) {
    static_assert(HD * (int)sizeof(T) == 16 * 64 && NK % NW == 0, "one wave instruction per key row");
    // wave wu stages key rows wu, wu + NW, ... of K and V; rows past the block's
    // keys read its first row (their scores are masked, their p is 0)
    const int wu = __builtin_amdgcn_readfirstlane(w);
    auto dma = [&](const Blk &d, int bf) {
#pragma unroll
      for (int i = 0; i < NK / NW; ++i) {
        const int r = wu + i * NW;
        const int64_t rr = r < d.rem ? r : 0;
        lds_row16(d.kb + rr * kv_stride + lane * VEC, Ks(bf) + r * KP);
        lds_row16(d.vb + rr * kv_stride + lane * VEC, Vt(bf) + r * VKP);
      }
    };
    // vmcnt(0), the other counters left alone (gfx9 encoding)
    constexpr int WAIT0 = (7 << 4) | (15 << 8);
    // block b is read from buffer b % 2 while block b+1 lands in the other one,
    // which every wave finished reading before the barrier that ended block b-1
    if (nb > 0) {
      dma(desc(0), 0);
      __builtin_amdgcn_s_waitcnt(WAIT0);
      __syncthreads();
    }
    for (int b = 0; b < nb; b += 2) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (b + j < nb) {
          if (b + j + 1 < nb) dma(desc(b + j + 1), (j + 1) % 2);
          __builtin_amdgcn_sched_barrier(0);
          if (live) compute(desc(b + j), j);
          __builtin_amdgcn_s_waitcnt(WAIT0);
          __syncthreads();
        }
      }
    }
  } else {
  if (nb > 0) {
#pragma unroll
    for (int j = 0; j < PF; ++j) fetch(desc(j), kr[j], vr[j]);
    stage(kr[0], vr[0], 0);
    fetch(desc(PF), kr[0], vr[0]);
    __syncthreads();
  }
  int b0 = 0;
  for (; b0 + U <= nb; b0 += U) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int b = b0 + j;
      __builtin_amdgcn_sched_barrier(0);
      if (live) compute(desc(b), j % 2);
      const int sl = (j + 1) % PF;
      stage(kr[sl], vr[sl], (j + 1) % 2);
      fetch(desc(b + 1 + PF), kr[sl], vr[sl]);
      __syncthreads();
    }
  }
#pragma unroll
  for (int j = 0; j < U - 1; ++j) {   // fewer than U blocks remain
    if (b0 + j < nb) {
      if (live) compute(desc(b0 + j), j % 2);
      const int sl = (j + 1) % PF;
      if (b0 + j + 1 < nb) stage(kr[sl], vr[sl], (j + 1) % 2);
      __syncthreads();
    }
  }
  }

  const int64_t R = (int64_t)a.nc * a.Hq * QN;
#pragma unroll
  for (int jb = 0; jb < QB; ++jb) {
    const int qi = cq[jb], hq = h + chd[jb];
    const int64_t cbq = cb + ccv[jb];   // the column's canvas
    const float L = group4_sum(grp == 0 ? oacc[HD / 16][jb][0] : 0.f);
    if (qi >= QN) continue;
    if (a.nsplit == 1) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      TO *o = static_cast<TO *>(a.o) + ((cbq * QN + qi) * a.Hq + hq) * HD;
#pragma unroll
      for (int rb = 0; rb < HD / 16; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[rb * 16 + grp * 4 + r] = from_f<TO>(oacc[rb][jb][r] * inv);
    } else {
      const int64_t row = (cbq * a.Hq + hq) * QN + qi;
      TO *po = static_cast<TO *>(a.part_o) + ((int64_t)s * R + row) * HD;
#pragma unroll
      for (int rb = 0; rb < HD / 16; ++rb) store4v<TO>(po + rb * 16 + grp * 4, oacc[rb][jb]);
      if (grp == 0) a.part_ml[(int64_t)s * R + row] = make_float2(mrun[jb], L);
    }
  }
}

// Fixed-order log-sum-exp merge of the split partials (scores in log2 units).
// One wave per output row, over the splits that hold keys of the row's query
// tile.  Pass 1 takes the maximum of the split maxima; pass 2 sums the weighted
// partials.  For HD = 64 a split's row is 16 float4 chunks, so the wave reads
// four splits per load (lane group g = lane / 16 takes splits g, g+4, ...) and
// the groups are added by a fixed butterfly; wider heads take one split per load.
// The same merge for few splits at head_dim 64: a 16-lane group per output row
// (its 16 float4 chunks), four rows per wave, each group over all the splits of
// its row in order.  One wave per row would leave most of its lanes idle and
// pay a wave's fixed cost per 64 outputs.
template <typename T, bool PREC = false>
__global__ __launch_bounds__(256) void attn_merge_rows_kernel(AttnArgs a) {
  using TO = typename std::conditional<PREC, float, T>::type;   // partial / output type
  constexpr int HD = 64, C4 = HD / 4;
  constexpr int NQ = AttnShape<T, HD>::NW * AttnShape<T, HD>::QB * 16;
  const int QN = a.qpos ? a.qn : a.C;
  const int64_t R = (int64_t)a.nc * a.Hq * QN;
  const int lane = threadIdx.x & 63;
  const int c0 = lane % C4;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= R) return;
  const int qi = (int)(row % QN);
  const int64_t ch = row / QN;
  const int h = (int)(ch % a.Hq);
  const int64_t cb = ch / a.Hq;
  if (a.active && !a.active[cb]) return;
  const int ncp = a.cpack > 1 ? a.cpack : 1;
  int64_t p0, plen;
  int lo, hi;
  tile_keys(a, (int)(cb / ncp * ncp), qi / NQ * NQ, NQ, &p0, &plen, &lo, &hi, ncp);
  const int64_t nk = plen + (hi - lo);
  const int ns = (int)(cdiv64(nk, a.chunk) < a.nsplit ? cdiv64(nk, a.chunk) : a.nsplit);
  const float2 *ml = a.part_ml + row;
  const TO *po = static_cast<const TO *>(a.part_o) + (row * C4 + c0) * 4;
  const int64_t sstride = R * C4 * 4;   // elements between splits
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[(int64_t)s * R].x);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY)
    for (int s = 0; s < ns; ++s) {
      const float2 v = ml[(int64_t)s * R];
      // raw v_exp_f32: the argument is <= 0 or -inf
      const float w = __builtin_amdgcn_exp2f(v.x - M);
      L += v.y * w;
      const float4 o = load4v<TO>(po + s * sstride);
      acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
    }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  TO *o = static_cast<TO *>(a.o) + ((cb * QN + qi) * a.Hq + h) * HD + 4 * c0;
  o[0] = from_f<TO>(acc.x * inv);
  o[1] = from_f<TO>(acc.y * inv);
  o[2] = from_f<TO>(acc.z * inv);
  o[3] = from_f<TO>(acc.w * inv);
}

template <typename T, int HD, bool PREC = false>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  using TO = typename std::conditional<PREC, float, T>::type;   // partial / output type
  constexpr int C4 = HD / 4;                     // float4 chunks per row
  constexpr int SG = C4 >= 64 ? 1 : 64 / C4;     // splits read side by side
  constexpr int CPL = C4 >= 64 ? C4 / 64 : 1;    // chunks per lane
  constexpr int NQ = AttnShape<T, HD>::NW * AttnShape<T, HD>::QB * 16;
  const int QN = a.qpos ? a.qn : a.C;
  const int64_t R = (int64_t)a.nc * a.Hq * QN;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  const int qi = (int)(row % QN);
  const int64_t ch = row / QN;
  const int h = (int)(ch % a.Hq);
  const int64_t cb = ch / a.Hq;
  if (a.active && !a.active[cb]) return;
  const int lane = threadIdx.x & 63;
  const int g = SG > 1 ? lane / C4 : 0;
  const int c0 = SG > 1 ? lane % C4 : lane;
  const int ncp = a.cpack > 1 ? a.cpack : 1;
  int64_t p0, plen;
  int lo, hi;
  tile_keys(a, (int)(cb / ncp * ncp), qi / NQ * NQ, NQ, &p0, &plen, &lo, &hi, ncp);
  const int64_t nk = plen + (hi - lo);
  const int ns = (int)(cdiv64(nk, a.chunk) < a.nsplit ? cdiv64(nk, a.chunk) : a.nsplit);
  const float2 *ml = a.part_ml + row;
  const TO *po = static_cast<const TO *>(a.part_o) + (row * C4 + c0) * 4;
  const int64_t sstride = R * C4 * 4;   // elements between splits

  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, ml[(int64_t)s * R].x);
#pragma unroll
  for (int off = 1; off < 64; off *= 2) M = fmaxf(M, __shfl_xor(M, off));
  float L = 0.f;
  float4 acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
#pragma unroll 4
    for (int s = g; s < ns; s += SG) {
      const float2 v = ml[(int64_t)s * R];
      // raw v_exp_f32: the argument is <= 0 or -inf
      const float w = __builtin_amdgcn_exp2f(v.x - M);
      L += v.y * w;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float4 o = load4v<TO>(po + s * sstride + 256 * c);
        acc[c].x += w * o.x; acc[c].y += w * o.y; acc[c].z += w * o.z; acc[c].w += w * o.w;
      }
    }
  }
  if constexpr (SG > 1) {
    // add the groups' sums (lanes c0 + C4 * g): partners combine the same two
    // values in the same order, so every group ends with identical sums
#pragma unroll
    for (int off = C4; off < 64; off *= 2) {
      const bool low = (lane & off) == 0;
      const float Lo = __shfl_xor(L, off);
      L = low ? L + Lo : Lo + L;
      float4 &x = acc[0];
      const float4 y = make_float4(__shfl_xor(x.x, off), __shfl_xor(x.y, off),
                                   __shfl_xor(x.z, off), __shfl_xor(x.w, off));
      x = low ? make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w)
              : make_float4(y.x + x.x, y.y + x.y, y.z + x.z, y.w + x.w);
    }
  }
  if (g != 0) return;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  TO *o = static_cast<TO *>(a.o) + ((cb * QN + qi) * a.Hq + h) * HD;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int d = 4 * (c0 + 64 * c);
    o[d + 0] = from_f<TO>(acc[c].x * inv);
    o[d + 1] = from_f<TO>(acc[c].y * inv);
    o[d + 2] = from_f<TO>(acc[c].z * inv);
    o[d + 3] = from_f<TO>(acc[c].w * inv);
  }
}

static_assert(AttnShape<bf16, 64>::NW * AttnShape<bf16, 64>::QB * 16 == 128 &&
              AttnShape<float, 64>::NW * AttnShape<float, 64>::QB * 16 == 128 &&
              AttnShape<bf16, 512>::NW * AttnShape<bf16, 512>::QB * 16 == 64,
              "query tile sizes");

// splits up to which the head_dim-64 merge takes a lane group per row
constexpr int kMergeRowsSplits = 8;

template <typename T, int HD, bool PREC, bool PATCH>
static hipError_t launch_attn_t(const AttnArgs &a, hipStream_t st) {
  constexpr int HKP = 4;   // kv heads a patched tile can serve together
  constexpr int NW = AttnShape<T, HD>::NW;
  constexpr int NQ = NW * AttnShape<T, HD>::QB * 16;
  const int QN = a.qpos ? a.qn : a.C;
  if (QN <= 0) return hipSuccess;
  AttnArgs b = a;
  const bool gathered = a.qpos != nullptr;
  // canvases packed in one tile must be consecutive in k, v (kv_cmul 1)
  const int cpp = a.kv_cmul > 1 ? 1 : a.canvas_per_prompt;
  b.cpack = attn_cpack(QN, gathered, a.Hq, a.Hkv, HD, cpp);
  b.packed = attn_packed(QN, gathered, a.Hq, a.Hkv, HD, cpp) ? 1 : 0;
  if (a.nc % b.cpack) return hipErrorInvalidValue;
  // patched tiles of 4 kv heads whose gathered queries fit a quarter tile each:
  // one workgroup for the four
  bool hk = false;
  if constexpr (PATCH && HD == 64 && sizeof(T) == 2)
    hk = a.Hkv == HKP && b.packed && (int64_t)(a.Hq / a.Hkv) * b.cpack * QN <= NQ / HKP;
  const dim3 grid = xcd_grid((int64_t)a.nc / b.cpack * (hk ? 1 : a.Hkv) * a.nsplit,
                             (hk || b.packed) ? 1 : (a.Hq / a.Hkv) * cdiv64(QN, NQ));
  if constexpr (PATCH && HD == 64 && sizeof(T) == 2) {
    if (hk) hipLaunchKernelGGL((attn_kernel<T, HD, PREC, PATCH, HKP>), grid, dim3(64 * NW), 0, st, b);
    else hipLaunchKernelGGL((attn_kernel<T, HD, PREC, PATCH>), grid, dim3(64 * NW), 0, st, b);
  } else {
    hipLaunchKernelGGL((attn_kernel<T, HD, PREC, PATCH>), grid, dim3(64 * NW), 0, st, b);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const int64_t R = (int64_t)a.nc * a.Hq * QN;
  if (HD == 64 && a.nsplit <= kMergeRowsSplits)
    hipLaunchKernelGGL((attn_merge_rows_kernel<T, PREC>), dim3((unsigned)cdiv64(R, 16)), dim3(256), 0, st, b);
  else
    hipLaunchKernelGGL((attn_merge_kernel<T, HD, PREC>), dim3((unsigned)cdiv64(R, 4)), dim3(256), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, int head_dim, bool bf, hipStream_t st) {
  if (a.prec && !bf) return hipErrorInvalidValue;
  const bool patch = a.kpatch != nullptr;
  // patched draws: gathered queries of canvases grouped by base canvas, k/v
  // not duplicated (kv_cmul 1), canvas lengths within the position map
  if (patch && (!attn_patch_supported(head_dim, bf, a.qn) || !a.prec || !a.qpos || a.kv_cmul > 1 || a.C > DG_MAX_CANVAS ||
                !a.vpatch || a.canvas_per_prompt < 1))
    return hipErrorInvalidValue;
  // encoder-mode chunks: every position of each chunk, one canvas per tile
  if (a.chunks && (a.qpos || patch || a.kv_cmul > 1 || a.canvas_per_prompt != 1))
    return hipErrorInvalidValue;
  if (bf && head_dim == 64) {
    if (patch) return a.prec ? launch_attn_t<bf16, 64, true, true>(a, st) : hipErrorInvalidValue;
    return a.prec ? launch_attn_t<bf16, 64, true, false>(a, st) : launch_attn_t<bf16, 64, false, false>(a, st);
  }
  if (bf && head_dim == 512)
    return a.prec ? launch_attn_t<bf16, 512, true, false>(a, st) : launch_attn_t<bf16, 512, false, false>(a, st);
  if (!bf && head_dim == 64) return launch_attn_t<float, 64, false, false>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace dg
