// The balanced work units of the decode attention's tiled kernels (built on the device).
#pragma once
#include "common.h"
#include "internal.h"

namespace mla {

// Work units of the tiled kernels for small batches, where contexts of different lengths would
// leave most fixed-length partitions of the short sequences empty.  Each sequence has p.splits
// partition slots; sequence b takes n_b = ceil(tiles_b / tps) of them.  tps starts at the
// shortest length that fits the longest sequence in its slots and is raised while that lowers
// the finish time, counted in rounds of p.cus units (one per compute unit) times tps.  The table
// lists the partitions in sequence order, then the slots no partition uses (p >= n_b: they get
// an empty partial, max -inf and no output rows), then B idle units: (b, p, first tile, end
// tile), b = -1 when idle.  One workgroup builds it from the lengths in device memory (B <= 64),
// so the host needs only B and splits.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// The builder takes one whole workgroup of 256 threads (it synchronises them once).
__device__ inline void build_decode_units(const DecodeAttnParams& p) {
  constexpr int kTile = 32;  // tokens per tile of the tiled kernels
  const int lane = threadIdx.x & 63;
  const int plus = p.lens_plus_one ? 1 : 0, S = p.splits, T = kTile;
  const int C = max(1, p.cus);
  // one lane per sequence (B <= 64)
  const int my_tiles = lane < p.B ? (p.lens[lane] + plus + T - 1) / T : 0;
  const int tot = wave_sum_int(my_tiles);
  int mx = my_tiles;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = max(mx, __shfl_xor(mx, d, 64));
  // partition length: the shortest one that fits every sequence in its S slots, or a longer one
  // when that finishes sooner; the finish time counts rounds of C units (one per compute unit)
  const int tmin = max(1, (mx + S - 1) / S);
  int tps = tmin;
  long best = -1;
  for (int k = 0; k <= 9; ++k) {
    const int cand = k < 9 ? tmin + tmin * k / 8 : max(tmin, (tot + C - 1) / C);
    const int used = wave_sum_int((my_tiles + cand - 1) / cand);
    const long cost = (long)((used + C - 1) / C) * cand;
    if (best < 0 || cost < best) {
      best = cost;
      tps = cand;
    }
  }
  // per-sequence partition counts and their prefix sums (B <= 64 here), then every thread fills
  // table entries
  __shared__ int s_tiles[64], s_pend[64], s_fend[64];  // tiles, partitions / free slots up to b
  if (threadIdx.x < 64) {
    const int tiles = my_tiles;
    const int n = lane < p.B ? (tiles + tps - 1) / tps : 0;
    s_tiles[lane] = tiles;
    s_pend[lane] = wave_incl_scan(n, lane);
    s_fend[lane] = wave_incl_scan(lane < p.B ? S - n : 0, lane);
  }
  __syncthreads();
  const int np = s_pend[p.B - 1];
  for (int j = threadIdx.x; j < p.B * S + p.B; j += blockDim.x) {
    int4 e = make_int4(-1, 0, 0, 0);
    if (j < np) {
      int i = 0;
      while (s_pend[i] <= j) ++i;
      const int k = j - (i ? s_pend[i - 1] : 0);
      e = make_int4(i, k, k * tps, min(s_tiles[i], (k + 1) * tps));
    } else if (j < p.B * S) {
      const int f = j - np;
      int i = 0;
      while (s_fend[i] <= f) ++i;
      const int n_i = s_pend[i] - (i ? s_pend[i - 1] : 0);
      e = make_int4(i, n_i + f - (i ? s_fend[i - 1] : 0), 0, 0);
    }
    p.units[j] = e;
  }
}


}  // namespace mla
