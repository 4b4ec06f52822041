// vs_aggregate.hip -- ground truth for the indexer: full causal attention
// weights summed along key columns and along diagonals, gfx950.
//
// VSPrefill (gist.science summaries of arXiv 2603.04460, English page,
// Technical Summary section 2, "Key Components, 2. Distillation Training,
// Ground Truth Generation"; German page, 2.B.2): the indexer is trained
// against attention weights aggregated per vertical column and per slash
// diagonal, computed block by block without materialising the n x n matrix.
//     a_v[g][j] = sum over query heads h of group g and rows i >= j of P^h_ij
//     a_s[g][o] = sum over h in g and rows i >= o of P^h_{i,i-o}
// P needs each row's final normaliser, so there are two passes:
//  1. dense causal attention (the sparse prefill kernel with every offset
//     selected) writes O and the row log-sum-exp;
//  2. this file's kernel recomputes S = Q K^T per 64-key tile, forms
//     P = exp2(S c - lse log2 e) in fp32, and adds it up: S is produced with
//     keys across lanes and rows across elements, so a column sum is a
//     per-lane add; diagonals go through LDS atomics into a ring indexed by
//     the offset.  After each tile the 64 column sums and the 64 diagonals no
//     later tile reaches leave through global atomics.
// The ring holds unsigned fixed point with 22 fraction bits: integer LDS
// atomics run at the rate of plain LDS stores on gfx950, while ds_add_f32 is
// several times slower.  A workgroup has 512 rows, so a ring slot (one
// diagonal) gathers at most 512 weights of at most 1 and stays below 2^32;
// each weight is rounded to nearest (error at most 2^-23), and the scale
// 2^22 is folded into the exponent.
#include <climits>
#include <type_traits>

#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

namespace {

constexpr int kAggWaves = 8;
constexpr int kAggThreads = kAggWaves * 64;
constexpr int kAggRows = 512;    // query rows (heads x positions) per workgroup
constexpr int kAggRing = 1024;   // diagonal ring entries (> positions + 127)
constexpr int kAggRingPad = 64;  // slots past the ring that alias its first 64
constexpr int kAggFrac = 22;     // fraction bits of the ring's fixed point
constexpr int kAggDmaWaves = 4;  // waves that load K tiles

struct AggParams {
  const void* q;
  const void* k;
  const float* lse;
  float* a_v;
  float* a_s;
  int n, hkv, group, bp, nblocks;
  float c;  // scale * log2(e)
};

// nearest integer of 0 <= x < 2^31 (halves round up); x + 0.5 is exact
// below 2^22, the range of the ring's terms
__device__ __forceinline__ uint32_t round_u32(float x) { return (uint32_t)(x + 0.5f); }

template <int D>
__device__ __forceinline__ int agg_swz(int r) {
  if constexpr (D == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

__global__ void agg_prepare_kernel(int32_t* s_off, int32_t* s_cnt, int32_t* v_idx, int32_t* v_cnt,
                                   float* a_v, float* a_s, int n) {
  const int g = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    s_off[(size_t)g * n + i] = i;
    a_v[(size_t)g * n + i] = 0.f;
    a_s[(size_t)g * n + i] = 0.f;
  }
  if (i == 0) {
    s_cnt[g] = n;
    v_idx[g] = -1;
    v_cnt[g] = 0;
  }
}

template <int D>
__global__ __launch_bounds__(kAggThreads) void agg_kernel(AggParams p) {
  constexpr int KS = D / 16;
  constexpr int CH = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = kBN * ROWB;
  constexpr int RPD = 1024 / ROWB;                 // key rows per 1 KiB DMA
  constexpr int NDMA = kBN / kAggDmaWaves / RPD;   // DMAs per loading wave per tile
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ __align__(16) uint8_t kt[2 * TILEB];
  __shared__ uint32_t ring[kAggRing + kAggRingPad];
  __shared__ float colp[kAggWaves][kBN];
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8* const kbase = (lds_u8*)kt;

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, ql = lane & 31;
  const int wave = wave_uniform(tid >> 6);
  const int n = p.n;
  const int g = blockIdx.x % p.hkv;
  const int b = p.nblocks - 1 - blockIdx.x / p.hkv;  // longest rows first
  const int i0 = b * p.bp;
  const int i1 = min(i0 + p.bp, n) - 1;
  const int groups_per_head = p.bp / 32;

  for (int t = tid; t < kAggRing + kAggRingPad; t += kAggThreads) ring[t] = 0u;

  // two row groups of 32 per wave: Q rows as the A operand, and per element
  // the bias that turns a logit into its weight times 2^kAggFrac
  bf16x8 qa[2][KS];
  float nls[2][16];
  int rbase[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int rg = wave * 2 + r;
    const int head = g * p.group + rg / groups_per_head;
    const int i0w = i0 + 32 * (rg % groups_per_head);
    rbase[r] = i0w;
    const int row = i0w + ql;
    const size_t ro = ((size_t)head * n + min(row, n - 1)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) + ro + 16 * s + 8 * half);
      if (row >= n) raw = u32x4{0u, 0u, 0u, 0u};
      qa[r][s] = as_bf16x8(raw);
    }
    // element 4a + bb holds row 8a + 4*half + bb of the group; rows past the
    // end get -inf, so their weights come out as exactly zero
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int ri = i0w + 8 * (e >> 2) + 4 * half + (e & 3);
      const float l = p.lse[(size_t)head * n + min(ri, n - 1)];
      nls[r][e] = ri < n ? (float)kAggFrac - l * kLog2e : -__builtin_inff();
    }
  }

  // LDS-DMA of one 64-key K tile (chunk-swizzled rows) by the first
  // kAggDmaWaves waves; the others never wait on vector memory, so the global
  // atomics they issue stay off the critical path
  const bool loader = wave < kAggDmaWaves;
  const u32x4 wk = buffer_words(static_cast<const char*>(p.k) + (size_t)g * n * ROWB, (uint32_t)(n * ROWB));
  int dma_row[NDMA], dma_col[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int r = (wave % kAggDmaWaves) * (kBN / kAggDmaWaves) + i * RPD + lane / CH;
    dma_row[i] = r;
    dma_col[i] = ((lane % CH) ^ agg_swz<D>(r)) * 16;
  }
  unsigned dma_off[NDMA];
  auto stage = [&](int tile, int st) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const unsigned off = (unsigned)(tile * kBN + dma_row[i]) * ROWB + dma_col[i];
      dma16(wk, (uint32_t)(uintptr_t)(kbase + st * TILEB +
                                      ((wave % kAggDmaWaves) * (kBN / kAggDmaWaves) + i * RPD) * ROWB),
            off);
      dma_off[i] = off;
    }
  };
  // Ring slot of element e of a 32x32 block: its offset row - key is
  // (rbase - key0 - 31) + lane_slot + erow(e), with erow(e) = 8(e/4) + e%4
  // and lane_slot = 4*half - ql + 31 in [0, 35]; the uniform part is taken
  // mod kAggRing, so a block's 63 slots are contiguous and may run up to
  // kAggRingPad slots past the ring, into the copies of its first slots
  const int lane_slot = 4 * half - ql + 31;
  int boff[KS];  // B operand: key row ql of a 32-key block, chunk 2s + half
#pragma unroll
  for (int s = 0; s < KS; ++s) boff[s] = ql * ROWB + 16 * ((2 * s + half) ^ agg_swz<D>(ql));

  // Key tiles are visited from a start tile that differs between workgroups,
  // wrapping round: workgroups that run at the same time then add into
  // different columns.  Diagonal offsets fall by kBN per tile within a run,
  // so after a tile the kBN largest offsets it touched are complete; at the
  // end of each run (the diagonal tile, and the last tile visited) every
  // offset still in the ring is.
  const int T = i1 / kBN + 1;
  const int t_first = (int)(((unsigned)b * 0x9E3779B1u + (unsigned)g * 0x7F4A7C15u) % (unsigned)T);
  const int diag_tile = i0 / kBN;  // first tile that needs the causal mask
  if (loader) stage(t_first, 0);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  __syncthreads();
  for (int it = 0; it < T; ++it) {
    const int t = t_first + it < T ? t_first + it : t_first + it - T;
    const int st = it & 1;
    if (loader && it + 1 < T) {
      stage(t + 1 < T ? t + 1 : 0, st ^ 1);
#pragma unroll
      for (int i = 0; i < NDMA; ++i) asm volatile("" ::"v"(dma_off[i]));
    }
    const int j0 = t * kBN;
    const lds_u8* kb = kbase + st * TILEB;
    float cs[2] = {0.f, 0.f};
    auto body = [&](auto masked) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int key = j0 + 32 * jb + ql;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          f32x16 s;
#pragma unroll
          for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) {
            const bf16x8 bo = *(const __attribute__((address_space(3))) bf16x8*)(kb + 32 * jb * ROWB + boff[kk]);
            s = mfma32(qa[r][kk], bo, s);
          }
          uint32_t* const slot = ring + ((rbase[r] - j0 - 32 * jb - 31) & (kAggRing - 1)) + lane_slot;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int erow = 8 * (e >> 2) + (e & 3);
            float pv = __builtin_amdgcn_exp2f(fmaf(s[e], p.c, nls[r][e]));
            if constexpr (decltype(masked)::value) pv = key <= rbase[r] + 4 * half + erow ? pv : 0.f;
            cs[jb] += pv;
            atomicAdd(slot + erow, round_u32(pv));
          }
        }
      }
    };
    if (t >= diag_tile) body(std::true_type{});
    else body(std::false_type{});
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      const float tot = half_sum(cs[jb]);
      if (half == 0) colp[wave][32 * jb + ql] = tot;
    }
    __syncthreads();
    const int top = i0 + p.bp - 1 - j0;  // largest offset this tile reaches
    if (wave == kAggDmaWaves) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kAggWaves; ++w) v += colp[w][lane];
      v *= 1.f / (float)(1 << kAggFrac);
      const int key = j0 + lane;
      if (key < n && v != 0.f) atomicAdd(&p.a_v[(size_t)g * n + key], v);
    } else if (wave == kAggDmaWaves + 1) {
      const bool run_end = t == T - 1 || it == T - 1;
      const int lo = run_end ? max(0, i0 - j0 - (kBN - 1)) : top - kBN + 1;
      for (int o = top - lane; o >= lo; o -= kBN) {
        if (o < 0 || o >= n) continue;
        const int sl = o & (kAggRing - 1);
        uint32_t u = ring[sl];
        ring[sl] = 0u;
        if (sl < kAggRingPad) {
          u += ring[kAggRing + sl];
          ring[kAggRing + sl] = 0u;
        }
        if (u != 0u) atomicAdd(&p.a_s[(size_t)g * n + o], (float)u * (1.f / (float)(1 << kAggFrac)));
      }
    }
    // the loaders' next tile has landed; the others only need their LDS work done
    if (loader) __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    else __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0)
    __syncthreads();
  }
}

int agg_positions(int group) { return kAggRows / group; }

}  // namespace

size_t aggregate_workspace_bytes(int h_kv, int n) {
  size_t o = align_up(sizeof(int32_t) * (size_t)h_kv * n, 256);  // offsets 0..n-1
  o += align_up(sizeof(int32_t) * 3 * (size_t)h_kv, 256);         // counts, empty column list
  return o + AttnWsLayout(h_kv, n, 1, n).total;
}

bool aggregate_grid_fits(int h_q, int h_kv, long long n) {
  const long long bp = agg_positions(h_q / h_kv);
  return (n + bp - 1) / bp * h_kv * kAggThreads < (1LL << 32) &&
         (n + 255) / 256 * 256 < (1LL << 32);
}

hipError_t launch_aggregate(const void* q, const void* k, const void* v, int h_q, int h_kv, int n,
                            int d, float scale, void* out, float* lse, float* a_v, float* a_s,
                            void* ws, hipStream_t stream) {
  char* base = static_cast<char*>(ws);
  int32_t* s_off = reinterpret_cast<int32_t*>(base);
  size_t o = align_up(sizeof(int32_t) * (size_t)h_kv * n, 256);
  int32_t* s_cnt = reinterpret_cast<int32_t*>(base + o);
  int32_t* v_idx = s_cnt + h_kv;
  int32_t* v_cnt = v_idx + h_kv;
  o += align_up(sizeof(int32_t) * 3 * (size_t)h_kv, 256);
  void* attn_ws = base + o;
  hipLaunchKernelGGL(agg_prepare_kernel, dim3((unsigned)((n + 255) / 256), (unsigned)h_kv), dim3(256),
                     0, stream, s_off, s_cnt, v_idx, v_cnt, a_v, a_s, n);
  AttnLayout dense;
  dense.full_tiles = true;  // every offset is selected
  hipError_t err = launch_attn(q, k, v, false, h_q, h_kv, n, d, scale, v_idx, v_cnt, 1, s_off, s_cnt, n,
                               out, lse, attn_ws, stream, dense);
  if (err != hipSuccess) return err;
  AggParams prm;
  prm.q = q;
  prm.k = k;
  prm.lse = lse;
  prm.a_v = a_v;
  prm.a_s = a_s;
  prm.n = n;
  prm.hkv = h_kv;
  prm.group = h_q / h_kv;
  prm.bp = agg_positions(prm.group);
  prm.nblocks = (n + prm.bp - 1) / prm.bp;
  prm.c = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)((long long)prm.nblocks * h_kv));
  if (d == 128) hipLaunchKernelGGL(agg_kernel<128>, grid, dim3(kAggThreads), 0, stream, prm);
  else hipLaunchKernelGGL(agg_kernel<64>, grid, dim3(kAggThreads), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace vs
