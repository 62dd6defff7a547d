// Expert grouping and the weighted combine of the MoE expert FFN on gfx950
// (the gather into expert-grouped rows and the "scatter with routing weights"
// steps of DEBUG_LOG.md "NVFP4 MoE Pipeline", "nvfp4-megamoe-kernel").
//
// route_kernel: one workgroup of 1024 threads (16 waves) turns topk_ids into
//   offsets[E+1]  exclusive prefix sum of the per-expert pair counts,
//   perm[P']      sorted position -> pair id, pairs grouped by expert and in
//                 increasing pair id inside each expert (stable, so the result
//                 is deterministic),
//   tiles[]       (expert, first sorted position, rows) for every block of up
//                 to `tile_rows` rows of one expert, and their count; with
//                 small_rows > 0, an expert's last block of at most
//                 small_rows rows goes to a second list (small[], *nsmall)
//                 for the GEMMs with short tiles instead.
// Each wave owns a contiguous range of pairs.  Pass 1 counts its pairs per
// expert in LDS; a prefix over (expert, wave) gives every wave its own
// starting position per expert; pass 2 re-reads the range 64 pairs at a time
// and ranks equal experts inside the wavefront with ballots on the expert id
// bits, so positions follow pair order without atomics on the output.
// Expert ids outside [0, E) are skipped and counted.
//
// For many pairs the same grouping runs over many workgroups (count, scan,
// place; below), with the same result.
//
// combine_kernel: y[t] = sum over j of o[t*k + j] in fixed order j = 0..k-1
// (each o row already carries alpha2 * routing weight).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteIdRegs = 4;  // steps of 64 pairs per wave whose ids one workgroup's grouping keeps in registers

// Exclusive prefix of v over the threads of the workgroup (one value per
// thread, kRouteThreads threads, scratch of at least 2 kRouteWaves ints);
// *total receives the sum.  Every thread must call it.  Each wave scans its
// 64 values with shuffles, the first wave scans the wave totals, and every
// thread adds its wave's offset: three barriers.
__device__ __forceinline__ int block_exclusive_scan(int* scan, int v, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) scan[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int t = lane < kRouteWaves ? scan[lane] : 0;
#pragma unroll
    for (int off = 1; off < kRouteWaves; off <<= 1) {
      const int y = __shfl_up(t, off, 64);
      if (lane >= off) t += y;
    }
    if (lane < kRouteWaves) scan[kRouteWaves + lane] = t;  // inclusive prefix of the wave totals
  }
  __syncthreads();
  const int base = wave ? scan[kRouteWaves + wave - 1] : 0;
  *total = scan[2 * kRouteWaves - 1];
  __syncthreads();  // the scratch is reused by the next call
  return base + x - v;
}

// Tiles of an expert with np rows: blocks of tile_rows rows; with
// small_rows > 0, a last block of at most small_rows rows goes on small
// tiles of small_tile rows instead (big: 0.., small: 0..).
struct TileCounts {
  int big, small;
};
__device__ __forceinline__ TileCounts tile_counts(int np, int tile_rows, int small_rows, int small_tile) {
  if (small_rows > 0) {
    const int r = np % tile_rows;
    return {np / tile_rows + (r > small_rows ? 1 : 0),
            (r > 0 && r <= small_rows) ? (r + small_tile - 1) / small_tile : 0};
  }
  return {(np + tile_rows - 1) / tile_rows, 0};
}

// Offsets, tile list and small-tile list of all experts, 1024 experts per
// chunk: count_of(e) gives expert e's pairs, on_start(e, start) hears its
// first sorted position.  Every thread must call it.
template <class CountOf, class OnStart>
__device__ __forceinline__ void group_tiles(int E, int tile_rows, int small_rows, int small_tile, int* scan,
                                            int* offsets, GemmTile* tiles, int* ntiles,
                                            GemmTile* small, int* nsmall, CountOf count_of,
                                            OnStart on_start) {
  const int tid = threadIdx.x;
  int base_p = 0, base_t = 0, base_s = 0;
  for (int e0 = 0; e0 < E; e0 += kRouteThreads) {
    const int e = e0 + tid;
    const int np = (e < E) ? count_of(e) : 0;
    const TileCounts c = tile_counts(np, tile_rows, small_rows, small_tile);
    int chunk_p, chunk_t, chunk_s;
    const int xp = block_exclusive_scan(scan, np, &chunk_p);
    const int xt = block_exclusive_scan(scan, c.big, &chunk_t);
    const int xs = block_exclusive_scan(scan, c.small, &chunk_s);
    if (e < E) {
      const int start = base_p + xp;
      offsets[e] = start;
      on_start(e, start);
      for (int k = 0; k < c.big; ++k)
        tiles[base_t + xt + k] = GemmTile{e, start + k * tile_rows, min(tile_rows, np - k * tile_rows), 0};
      for (int k = 0; k < c.small; ++k) {
        const int r0 = c.big * tile_rows + k * small_tile;
        small[base_s + xs + k] = GemmTile{e, start + r0, min(small_tile, np - r0), 0};
      }
    }
    base_p += chunk_p;
    base_t += chunk_t;
    base_s += chunk_s;
  }
  if (tid == 0) {
    offsets[E] = base_p;
    *ntiles = base_t;
    if (nsmall) *nsmall = base_s;
  }
}

// The grouping in one workgroup of kRouteThreads threads; sm is its LDS
// (route_lds_bytes(E)).
__device__ __forceinline__ void route_block(int* sm, int& s_err, const int32_t* __restrict__ ids, int64_t P,
                                            int E, int tile_rows, int small_rows, int small_tile,
                                            int* __restrict__ offsets, int* __restrict__ perm,
                                            GemmTile* __restrict__ tiles, int* __restrict__ ntiles,
                                            GemmTile* __restrict__ small, int* __restrict__ nsmall,
                                            int* __restrict__ err_count, int* __restrict__ sched) {
  int* cnt = sm;                            // [waves][E]: pass-1 counts, then running positions
  int* total = cnt + kRouteWaves * E;       // [E]
  int* scan = total + E;                    // [1024] block scan scratch

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // wave w owns pairs [p0, p1), 64 per step; the ids of its first
  // kRouteIdRegs steps are loaded once, before anything else (both passes
  // use them), the rest of a larger range is read in each pass
  const int64_t p0 = P * wave / kRouteWaves, p1 = P * (wave + 1) / kRouteWaves;
  int idr[kRouteIdRegs];
#pragma unroll
  for (int c = 0; c < kRouteIdRegs; ++c) {
    const int64_t p = p0 + 64 * c + lane;
    idr[c] = p < p1 ? ids[p] : -1;
  }
  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) cnt[i] = 0;
  if (tid == 0) s_err = 0;
  __syncthreads();

  int* mycnt = cnt + wave * E;
  auto count = [&](int64_t p, int e) {
    if (p >= p1) return;
    if (e >= 0 && e < E)
      atomicAdd(&mycnt[e], 1);
    else
      atomicAdd(&s_err, 1);
  };
#pragma unroll
  for (int c = 0; c < kRouteIdRegs; ++c) count(p0 + 64 * c + lane, idr[c]);
  for (int64_t p = p0 + 64 * kRouteIdRegs + lane; p < p1; p += 64) count(p, ids[p]);
  __syncthreads();

  // per expert: total, and each wave's start relative to the expert start
  for (int e = tid; e < E; e += kRouteThreads) {
    int run = 0;
    for (int w = 0; w < kRouteWaves; ++w) {
      int c = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += c;
    }
    total[e] = run;
  }
  __syncthreads();

  group_tiles(E, tile_rows, small_rows, small_tile, scan, offsets, tiles, ntiles, small, nsmall,
              [&](int e) { return total[e]; },
              [&](int e, int start) {
                for (int w = 0; w < kRouteWaves; ++w) cnt[w * E + e] += start;
              });
  __syncthreads();
  if (tid == 0 && err_count) *err_count = s_err;
  if (sched && tid < kSchedCounters) sched[tid] = 0;

  // pass 2: stable placement, 64 pairs per step, ranks by ballot matching
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // one step of 64 pairs (e = -1 past the range; every lane takes part)
  auto place = [&](int64_t p, int e) {
    const bool valid = e >= 0 && e < E;
    uint64_t match = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      uint64_t ones = __ballot(valid && ((e >> bit) & 1));
      match &= ((e >> bit) & 1) ? ones : ~ones;
    }
    if (valid) {
      const int rank = __popcll(match & lt_mask);
      const int pos = mycnt[e] + rank;
      perm[pos] = (int)p;
      if ((match & lt_mask) == 0) mycnt[e] = pos - rank + __popcll(match);
    }
  };
#pragma unroll
  for (int c = 0; c < kRouteIdRegs; ++c)
    if (p0 + 64 * c < p1) place(p0 + 64 * c + lane, idr[c]);
  for (int64_t b = p0 + 64 * kRouteIdRegs; b < p1; b += 64) {
    const int64_t p = b + lane;
    place(p, (p < p1) ? ids[p] : -1);
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(const int32_t* __restrict__ ids,
                                                              int64_t P, int E, int tile_rows,
                                                              int small_rows, int small_tile,
                                                              int* __restrict__ offsets,
                                                              int* __restrict__ perm,
                                                              GemmTile* __restrict__ tiles,
                                                              int* __restrict__ ntiles,
                                                              GemmTile* __restrict__ small,
                                                              int* __restrict__ nsmall,
                                                              int* __restrict__ err_count,
                                                              int* __restrict__ sched) {
  extern __shared__ int sm[];
  __shared__ int s_err;
  route_block(sm, s_err, ids, P, E, tile_rows, small_rows, small_tile, offsets, perm, tiles, ntiles, small,
              nsmall, err_count, sched);
}

// The grouping (workgroup 0, as route_kernel) and, independent of it, the
// first pass of the activations' global scale (workgroups 1 .. namax: the
// maximum of |x| over a grid-stride range of 8-element chunks each, into
// partial[0 .. namax)): one launch instead of two, the grouping running
// beside the maxima.
__global__ __launch_bounds__(kRouteThreads) void amax_route_kernel(const uint4* __restrict__ x, int64_t n8,
                                                                   float* __restrict__ partial, int namax,
                                                                   const int32_t* __restrict__ ids,
                                                                   int64_t P, int E, int tile_rows,
                                                                   int small_rows, int small_tile,
                                                                   int* __restrict__ offsets,
                                                                   int* __restrict__ perm,
                                                                   GemmTile* __restrict__ tiles,
                                                                   int* __restrict__ ntiles,
                                                                   GemmTile* __restrict__ small,
                                                                   int* __restrict__ nsmall,
                                                                   int* __restrict__ err_count,
                                                                   int* __restrict__ sched) {
  extern __shared__ int sm[];
  __shared__ int s_err;
  if (blockIdx.x == 0) {
    route_block(sm, s_err, ids, P, E, tile_rows, small_rows, small_tile, offsets, perm, tiles, ntiles, small,
                nsmall, err_count, sched);
    return;
  }
  const int b = (int)blockIdx.x - 1, tid = threadIdx.x;
  float m = 0.0f;
  for (int64_t i = (int64_t)b * kRouteThreads + tid; i < n8; i += (int64_t)namax * kRouteThreads) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + i));  // read once
    m = fmaxf(m, abs_max8(make_uint4(v.x, v.y, v.z, v.w)));
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float* red = reinterpret_cast<float*>(sm);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    float r = red[0];
    for (int w = 1; w < kRouteWaves; ++w) r = fmaxf(r, red[w]);
    partial[b] = r;
  }
}

// ---- the same grouping over many workgroups (large P).  Workgroup g of G
// owns pairs [P g / G, P (g + 1) / G).  route_count_kernel counts each
// workgroup's pairs per expert; route_scan_kernel turns the counts into each
// workgroup's first position per expert (experts in order, workgroups in
// order inside an expert), the offsets and the tile list;
// route_place_kernel places each workgroup's pairs as the single-workgroup
// kernel does, so perm is the same stable order.

__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(const int32_t* __restrict__ ids,
                                                                    int64_t P, int E,
                                                                    int* __restrict__ gcount,
                                                                    int* __restrict__ gerr) {
  extern __shared__ int cnt[];  // [E]
  __shared__ int s_err;
  const int tid = threadIdx.x, G = gridDim.x, g = blockIdx.x;
  for (int e = tid; e < E; e += kRouteThreads) cnt[e] = 0;
  if (tid == 0) s_err = 0;
  __syncthreads();
  const int64_t p0 = P * g / G, p1 = P * (g + 1) / G;
  for (int64_t p = p0 + tid; p < p1; p += kRouteThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E)
      atomicAdd(&cnt[e], 1);
    else
      atomicAdd(&s_err, 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) gcount[(int64_t)g * E + e] = cnt[e];
  if (tid == 0) gerr[g] = s_err;
}

__global__ __launch_bounds__(kRouteThreads) void route_scan_kernel(int G, int E, int tile_rows,
                                                                   int small_rows, int small_tile,
                                                                   int* __restrict__ gcount,
                                                                   const int* __restrict__ gerr,
                                                                   int* __restrict__ offsets,
                                                                   GemmTile* __restrict__ tiles,
                                                                   int* __restrict__ ntiles,
                                                                   GemmTile* __restrict__ small,
                                                                   int* __restrict__ nsmall,
                                                                   int* __restrict__ err_count,
                                                                   int* __restrict__ sched) {
  __shared__ int scan[kRouteThreads];
  const int tid = threadIdx.x;
  // each expert's pairs per workgroup -> exclusive starts within the expert,
  // then (with the expert's start) the workgroup's first position per expert
  group_tiles(E, tile_rows, small_rows, small_tile, scan, offsets, tiles, ntiles, small, nsmall,
              [&](int e) {
                int np = 0;
                for (int g = 0; g < G; ++g) {
                  const int c = gcount[(int64_t)g * E + e];
                  gcount[(int64_t)g * E + e] = np;
                  np += c;
                }
                return np;
              },
              [&](int e, int start) {
                for (int g = 0; g < G; ++g) gcount[(int64_t)g * E + e] += start;
              });
  if (tid == 0) {
    int err = 0;
    for (int g = 0; g < G; ++g) err += gerr[g];
    if (err_count) *err_count = err;
  }
  if (sched && tid < kSchedCounters) sched[tid] = 0;
}

__global__ __launch_bounds__(kRouteThreads) void route_place_kernel(const int32_t* __restrict__ ids,
                                                                    int64_t P, int E,
                                                                    const int* __restrict__ gcount,
                                                                    int* __restrict__ perm) {
  extern __shared__ int cnt[];  // [waves][E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, G = gridDim.x, g = blockIdx.x;
  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) cnt[i] = 0;
  __syncthreads();
  const int64_t q0 = P * g / G, q1 = P * (g + 1) / G, n = q1 - q0;
  const int64_t p0 = q0 + n * wave / kRouteWaves, p1 = q0 + n * (wave + 1) / kRouteWaves;
  int* mycnt = cnt + wave * E;
  for (int64_t p = p0 + lane; p < p1; p += 64) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&mycnt[e], 1);
  }
  __syncthreads();
  // each wave's first position per expert: the workgroup's start plus the
  // pairs of the earlier waves
  for (int e = tid; e < E; e += kRouteThreads) {
    int run = gcount[(int64_t)g * E + e];
    for (int w = 0; w < kRouteWaves; ++w) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t b = p0; b < p1; b += 64) {
    const int64_t p = b + lane;
    const int e = (p < p1) ? ids[p] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t match = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t ones = __ballot(valid && ((e >> bit) & 1));
      match &= ((e >> bit) & 1) ? ones : ~ones;
    }
    if (valid) {
      const int rank = __popcll(match & lt_mask);
      const int pos = mycnt[e] + rank;
      perm[pos] = (int)p;
      if ((match & lt_mask) == 0) mycnt[e] = pos - rank + __popcll(match);
    }
  }
}

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o,
                                                      const int32_t* __restrict__ ids, int E,
                                                      int64_t T, int k, int64_t H,
                                                      void* __restrict__ out) {
  const int64_t n4 = H / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < T * n4;
       i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / n4, c = (i % n4) * 4;
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int e = ids[t * k + j];
      if (e < 0 || e >= E) continue;
      const float4 v = *reinterpret_cast<const float4*>(o + (t * k + j) * H + c);
      y.x += v.x;
      y.y += v.y;
      y.z += v.z;
      y.w += v.w;
    }
    if (BF16_OUT) {
      __bf16 h[4] = {(__bf16)y.x, (__bf16)y.y, (__bf16)y.z, (__bf16)y.w};
      uint2 u;
      __builtin_memcpy(&u, h, 8);
      reinterpret_cast<uint2*>(out)[(t * H + c) / 4] = u;
    } else {
      reinterpret_cast<float4*>(out)[(t * H + c) / 4] = y;
    }
  }
}

// The same sum over the f16 form of o: o16[r][c] * 2^oexp[r][c / 32] (exact
// in fp32), 8 columns per thread.  With k <= KMAX the k expert ids and then
// the k rows are all loaded before the first addition (streaming loads: each
// row is read once), so a thread keeps k loads in flight; the sum still runs
// in the fixed order j = 0 .. k - 1.  KMAX = 0: a plain loop for any k.
template <bool BF16_OUT, int KMAX>
__global__ __launch_bounds__(256) void combine_f16_kernel(const uint16_t* __restrict__ o16,
                                                          const int8_t* __restrict__ oexp,
                                                          const int32_t* __restrict__ ids, int E,
                                                          int64_t T, int k, int64_t H,
                                                          void* __restrict__ out) {
  const int64_t n8 = H / 8, nb = H / 32;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < T * n8;
       i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / n8, c = (i % n8) * 8;
    float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto add = [&](const uint4& v, int s) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        y[2 * q] += ldexpf((float)__builtin_bit_cast(_Float16, (uint16_t)(w[q] & 0xffffu)), s);
        y[2 * q + 1] += ldexpf((float)__builtin_bit_cast(_Float16, (uint16_t)(w[q] >> 16)), s);
      }
    };
    if (KMAX > 0) {
      bool ok[KMAX > 0 ? KMAX : 1];
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const int e = j < k ? ids[t * k + j] : -1;
        ok[j] = e >= 0 && e < E;
      }
      uint4 v[KMAX > 0 ? KMAX : 1];
      int s[KMAX > 0 ? KMAX : 1];
      // every row of the token is loaded together with the ids (rows of
      // skipped pairs hold stale bytes and are not added): one round trip
      // to memory instead of two
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const int64_t r = t * k + j;
        if (j < k) {  // kernel-uniform
          const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o16 + r * H + c));
          v[j] = make_uint4(x.x, x.y, x.z, x.w);
          s[j] = oexp[r * nb + c / 32];
        } else {
          v[j] = make_uint4(0, 0, 0, 0);
          s[j] = 0;
        }
      }
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (ok[j]) add(v[j], s[j]);
    } else {
      for (int j = 0; j < k; ++j) {
        const int64_t r = t * k + j;
        const int e = ids[r];
        if (e < 0 || e >= E) continue;
        add(*reinterpret_cast<const uint4*>(o16 + r * H + c), oexp[r * nb + c / 32]);
      }
    }
    if (BF16_OUT) {
      __bf16 h[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) h[q] = (__bf16)y[q];
      u32x4 u;
      __builtin_memcpy(&u, h, 16);
      __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(out) + (t * H + c) / 8);
    } else {
      float4* dst = reinterpret_cast<float4*>(out) + (t * H + c) / 4;
      dst[0] = make_float4(y[0], y[1], y[2], y[3]);
      dst[1] = make_float4(y[4], y[5], y[6], y[7]);
    }
  }
}

size_t route_lds_bytes(int E) { return sizeof(int) * ((size_t)kRouteWaves * E + E + kRouteThreads); }

// Pairs per workgroup of the many-workgroup grouping, and the most workgroups.
constexpr int64_t kRouteChunk = 4096;
constexpr int kAmaxRouteMax = 256;  // maxima of the fused global-scale pass, at most
constexpr int kRouteMaxGroups = 256;

int route_groups(int64_t P) {
  const int64_t g = (P + kRouteChunk - 1) / kRouteChunk;
  return (int)(g < 1 ? 1 : g > kRouteMaxGroups ? kRouteMaxGroups : g);
}

size_t route_workspace_bytes(int64_t P, int E) {
  const int G = route_groups(P);
  return sizeof(int) * ((size_t)G * E + G);
}

hipError_t launch_route(const int32_t* ids, int64_t P, int E, int tile_rows, int small_rows, int small_tile,
                        int* offsets,
                        int* perm, GemmTile* tiles, int* ntiles, GemmTile* small, int* nsmall, int* err_count,
                        int* ws, int* sched, hipStream_t s) {
  const int G = route_groups(P);
  if (G == 1 || !ws) {
    route_kernel<<<1, kRouteThreads, route_lds_bytes(E), s>>>(ids, P, E, tile_rows, small_rows, small_tile,
                                                              offsets, perm,
                                                              tiles, ntiles, small, nsmall, err_count, sched);
    return hipGetLastError();
  }
  int* gcount = ws;
  int* gerr = ws + (size_t)G * E;
  route_count_kernel<<<G, kRouteThreads, sizeof(int) * E, s>>>(ids, P, E, gcount, gerr);
  route_scan_kernel<<<1, kRouteThreads, 0, s>>>(G, E, tile_rows, small_rows, small_tile, gcount, gerr, offsets,
                                                 tiles, ntiles,
                                                 small, nsmall, err_count, sched);
  route_place_kernel<<<G, kRouteThreads, sizeof(int) * kRouteWaves * E, s>>>(ids, P, E, gcount, perm);
  return hipGetLastError();
}

bool route_single(int64_t P) { return route_groups(P) == 1; }

int amax_route_blocks(int64_t n8) {
  const int64_t b = (n8 + 4 * kRouteThreads - 1) / (4 * kRouteThreads);
  return (int)(b < 1 ? 1 : b > kAmaxRouteMax ? kAmaxRouteMax : b);
}

hipError_t launch_amax_route(const uint16_t* x, int64_t n, float* partial, int namax, const int32_t* ids,
                             int64_t P, int E, int tile_rows, int small_rows, int small_tile, int* offsets,
                             int* perm, GemmTile* tiles, int* ntiles, GemmTile* small, int* nsmall,
                             int* err_count, int* sched, hipStream_t s) {
  if (!route_single(P) || namax < 1 || namax > kAmaxRouteMax) return hipErrorInvalidValue;
  amax_route_kernel<<<namax + 1, kRouteThreads, route_lds_bytes(E), s>>>(
      reinterpret_cast<const uint4*>(x), n / 8, partial, namax, ids, P, E, tile_rows, small_rows, small_tile,
      offsets, perm, tiles, ntiles, small, nsmall, err_count, sched);
  return hipGetLastError();
}

hipError_t launch_combine(const float* o, const int32_t* ids, int E, int64_t T, int k, int64_t H,
                          bool bf16_out, void* out, hipStream_t s, const uint16_t* o_f16,
                          const int8_t* o_exp) {
  if (o_f16) {
    const int64_t n = T * (H / 8);
    if (n == 0) return hipSuccess;
    const int64_t wg = std::min<int64_t>((n + 255) / 256, 65536);
    if (k <= 8) {
      if (bf16_out)
        combine_f16_kernel<true, 8><<<(unsigned)wg, 256, 0, s>>>(o_f16, o_exp, ids, E, T, k, H, out);
      else
        combine_f16_kernel<false, 8><<<(unsigned)wg, 256, 0, s>>>(o_f16, o_exp, ids, E, T, k, H, out);
    } else if (bf16_out) {
      combine_f16_kernel<true, 0><<<(unsigned)wg, 256, 0, s>>>(o_f16, o_exp, ids, E, T, k, H, out);
    } else {
      combine_f16_kernel<false, 0><<<(unsigned)wg, 256, 0, s>>>(o_f16, o_exp, ids, E, T, k, H, out);
    }
    return hipGetLastError();
  }
  int64_t n = T * (H / 4);
  if (n == 0) return hipSuccess;
  int64_t wg = (n + 255) / 256;
  if (wg > 65536) wg = 65536;
  if (bf16_out)
    combine_kernel<true><<<(unsigned)wg, 256, 0, s>>>(o, ids, E, T, k, H, out);
  else
    combine_kernel<false><<<(unsigned)wg, 256, 0, s>>>(o, ids, E, T, k, H, out);
  return hipGetLastError();
}

}  // namespace nvfp4
