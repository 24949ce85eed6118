// Host-side planning of the launches: split counts, tile sizes and the
// split-KV plan of attention.  Plain host code (no kernels), shared by the
// launchers and by the workspace queries of the C-ABI layer.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dg {

// Projections at small M are weight-streaming and latency-bound: 64 x 64 tiles
// with a 4-stage prefetch, and below 256 tiles the K range is split so that
// about 512 workgroups stream the weights (the bf16 path; K splits of at least
// 512).  Partials are summed by a separate reduce in split order.  Measured at
// d 2816: the read's projections of 40 slot rows take 15-17.5 instead of 19-27
// us; splitting the step's 384-tile q,k,v projection in two, or its output
// projection in five, was no faster (each extra launch costs about 4 us).
void proj_split(int64_t M, int64_t ncols, int K, bool bf, int *ks, int *kchunk) {
  *ks = 1;
  *kchunk = K;
  if (!bf || M <= 0 || ncols <= 0 || K <= 0) return;
  const int64_t tiles = cdiv64(M, 64) * cdiv64(ncols, 64);
  if (tiles >= 256) return;
  int64_t s = 512 / tiles;
  if (s > K / 512) s = K / 512;
  if (s < 2) return;
  const int64_t steps = cdiv64(K, 64), per = cdiv64(steps, s);
  *ks = (int)cdiv64(steps, per);
  *kchunk = (int)(per * 64);
}

int proj_ksplit(int64_t M, int64_t ncols, int K, bool bf) {
  int ks, kc;
  proj_split(M, ncols, K, bf, &ks, &kc);
  return ks;
}

// Vocabulary ranges of the self-conditioning GEMM: about one workgroup per CU
// (with XCD grouping: as many whole ranges per XCD as fit its 32 CUs).
int sc_ksplit(int64_t M, int d, int vocab, bool bf) {
  const int64_t tiles = bf ? cdiv64(M, 256) * cdiv64(d, kScTileD) : cdiv64(M, 64) * cdiv64(d, 64);
  if (tiles <= 0) return 1;   // no rows: nothing to split
  const int nk = vocab / (bf ? 64 : 16);
  const int64_t per_xcd = 32 / tiles;
  int64_t ks = kScGroup ? (per_xcd >= 1 ? 8 * per_xcd : 8) : 256 / tiles;
  if (ks > nk) ks = nk;
  if (ks > 64) ks = 64;
  // bf16: once about 128 workgroups run, each split spans at least 512
  // vocabulary entries (16 K steps of the direct-to-LDS loop), so short loops
  // do not trade their work for fp32 partial-sum traffic (ragged batch of 32
  // canvases: 8 -> 4 splits, 39 -> 35 us)
  if (bf) {
    const int64_t cap = std::max<int64_t>(vocab / 512, cdiv64(128, tiles));
    if (ks > cap) ks = cap;
  }
  if (ks < 1) ks = 1;
  return (int)ks;
}

int attn_query_tile(int head_dim) { return head_dim == 512 ? 64 : 128; }

int attn_cpack(int qn, bool gathered, int Hq, int Hkv, int head_dim, int cpp) {
  if (!gathered || cpp <= 1) return 1;
  return (int64_t)cpp * (Hq / Hkv) * qn <= attn_query_tile(head_dim) ? cpp : 1;
}

bool attn_packed(int qn, bool gathered, int Hq, int Hkv, int head_dim, int cpp) {
  if (!gathered) return false;
  if (attn_cpack(qn, gathered, Hq, Hkv, head_dim, cpp) > 1) return true;
  return Hq > Hkv && (int64_t)(Hq / Hkv) * qn <= attn_query_tile(head_dim);
}
void attn_plan(int nc, int C, int qn, bool gathered, int Hq, int Hkv, int W, int head_dim,
               int max_len, int cpp, int *nsplit, int *chunk, int *nsplit_bound) {
  const int nq = attn_query_tile(head_dim);
  const int nk = head_dim == 512 ? 32 : 64;
  const int ncp = attn_cpack(qn, gathered, Hq, Hkv, head_dim, cpp);
  const int64_t base = attn_packed(qn, gathered, Hq, Hkv, head_dim, cpp)
                           ? (int64_t)nc / ncp * Hkv
                           : (int64_t)nc * Hq * cdiv64(qn, nq);
  // most keys one query tile can see: the prompt plus its window span (every
  // canvas key of the tile's canvases for gathered queries)
  // (patched tiles: at most C base rows and ncp * qn slot rows)
  const int64_t win = gathered ? std::max<int64_t>((int64_t)C * ncp, (int64_t)C + (int64_t)ncp * qn)
                               : (nq + 2 * (int64_t)W < C ? nq + 2 * (int64_t)W : C);
  const int64_t span = (int64_t)max_len + win;
  // about two workgroups per CU at head_dim 64; at head_dim 512 one (its 135 KB
  // of LDS leaves room for one), so each CU runs a single workgroup with twice
  // the key blocks instead of two in turn, paying its prologue and epilogue once
  // (headline step: 54 -> 42 us)
  const int target = head_dim == 512 ? 256 : 512;
  int ns = 1;
  if (base > 0 && base < target) {   // (no tiles at all: nothing to split)
    ns = (int)cdiv64(target, base);
    const int64_t maxs = cdiv64(span, 4 * nk);   // keep at least ~4 key blocks per split
    if (ns > maxs) ns = (int)maxs;
    if (ns < 1) ns = 1;
  }
  // ns is non-decreasing in max_len; the rounded count below never exceeds it,
  // so ns bounds the splits of every prompt up to max_len (workspace sizing)
  if (nsplit_bound) *nsplit_bound = ns;
  const int ck = (int)(cdiv64(cdiv64(span, ns), nk) * nk);
  ns = (int)cdiv64(span, ck);
  if (ns < 1) ns = 1;
  *nsplit = ns;
  *chunk = ck;
}

// (a patched tile keeps its canvas keys -- at most C base rows and cpack * qn
// slot rows, qn <= C -- in a table of 2 DG_MAX_CANVAS entries)
bool attn_patch_supported(int head_dim, bool bf, int n_slots) {
  return bf && head_dim == 64 && n_slots >= 0 && n_slots <= DG_MAX_CANVAS;
}

}  // namespace dg
