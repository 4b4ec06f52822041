// vs_attn.hip -- index-to-tile builder and vertical-slash sparse prefill
// attention for gfx950 (MI355X).
//
// What is computed (VSPrefill, gist.science summaries of arXiv 2603.04460:
// English page, Technical Summary section 2, "Core Concept: Vertical-Slash
// Pattern" and "3. Adaptive Inference Pipeline, Fused Kernel Execution";
// German page section 2.A gives the slash as the relative shift i - j):
// for query head h of KV group g and row i, attention over
//     S_i = { j <= i : j in V_g  or  i - j in O_g }.
//
// How it is laid out on the chip
//  * Builder (4 tiny launches per call): per KV head, bitmaps of the
//    selected offsets and columns, a per-word prefix count of the offset
//    bitmap, sorted duplicate-free lists, and "clusters": maximal runs of
//    sorted offsets whose gaps are small enough that, for a block of BMP
//    query rows, the keys they reach form one contiguous range of key tiles.
//  * Attention: one workgroup per (KV head, block of BMP query positions);
//    its waves are the G query heads of the group (and, for G < 4, several
//    32-row sub-blocks), so every K/V tile staged in LDS feeds all G heads.
//    The sorted cluster list is walked from the largest offset down, which
//    yields the key-tile ranges of the block in ascending key order (a merge
//    of the per-cluster ranges, no n x n structure).  Each contiguous tile is
//    masked per element by (j <= i) and (offset bit or column bit); the lane
//    masks come from wave-uniform bitmap windows, so a masked element costs
//    one v_cndmask.  Columns that no processed tile covers are then gathered
//    64 at a time into tiles of their own.
//  * Math per 64-key tile and 32 query rows: S^T = K Q^T on
//    v_mfma_f32_32x32x16_bf16 (K from LDS, Q^T held in registers), online
//    softmax in fp32 on the transposed scores (each lane owns one query row,
//    so row statistics need one cross-half exchange), P^T reused directly as
//    the B operand of O^T += V^T P^T with V^T staged in LDS in a matching
//    key order.  The running maximum is only moved when it grows by more
//    than 2^8 (the result is unchanged; p stays below 2^8 in fp32/bf16).
#include <algorithm>
#include <climits>

#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

namespace {

constexpr float kTau = 8.0f;            // lazy-rescale threshold, log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNoMax = -1.0e30f;      // running max before any key was seen

// ---------------------------------------------------------------- builder

template <int NT>
__device__ int block_excl_scan(int v, int* total, int* sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  constexpr int NWV = NT / 64;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int t = lane < NWV ? sh[lane] : 0;
    int s = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    if (lane < NWV) sh[lane] = s - t;
    if (lane == NWV - 1) sh[NWV] = s;
  }
  __syncthreads();
  int res = sh[wv] + x - v;
  *total = sh[NWV];
  __syncthreads();
  return res;
}

__global__ void ws_clear_kernel(uint32_t* bitO, uint32_t* bitV, size_t nwords,
                                unsigned long long* stats) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t step = (size_t)gridDim.x * blockDim.x;
  for (; i < nwords; i += step) {
    bitO[i] = 0u;
    bitV[i] = 0u;
  }
  if (blockIdx.x == 0 && threadIdx.x < 4) stats[threadIdx.x] = 0ull;
}

__global__ void ws_setbits_kernel(const int32_t* __restrict__ v_idx, const int32_t* __restrict__ v_cnt,
                                  int cap_v, const int32_t* __restrict__ s_off,
                                  const int32_t* __restrict__ s_cnt, int cap_s, int n,
                                  uint32_t* bitO, uint32_t* bitV, int stride) {
  const int g = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int cv = min(max(v_cnt[g], 0), cap_v);
  const int cs = min(max(s_cnt[g], 0), cap_s);
  if (t < cv) {
    int x = v_idx[(size_t)g * cap_v + t];
    if (x >= 0 && x < n) atomicOr(&bitV[(size_t)g * stride + kPrePad + (x >> 5)], 1u << (x & 31));
  }
  if (t < cs) {
    int x = s_off[(size_t)g * cap_s + t];
    if (x >= 0 && x < n) atomicOr(&bitO[(size_t)g * stride + kPrePad + (x >> 5)], 1u << (x & 31));
  }
}

// per head: prefix counts of the offset bitmap and sorted unique lists
__global__ __launch_bounds__(1024) void ws_scan_kernel(const uint32_t* __restrict__ bitO,
                                                       const uint32_t* __restrict__ bitV,
                                                       int stride, int words, uint32_t* prefO,
                                                       int32_t* cleanO, int cap_s,
                                                       int32_t* cleanV, int cap_v,
                                                       int32_t* counts) {
  __shared__ int sh[17];
  const int g = blockIdx.x, tid = threadIdx.x;
  const uint32_t* bo = bitO + (size_t)g * stride + kPrePad;
  const uint32_t* bv = bitV + (size_t)g * stride + kPrePad;
  const int per = (words + 1023) / 1024;
  const int w0 = min(tid * per, words), w1 = min(w0 + per, words);
  int co = 0, cv = 0;
  for (int w = w0; w < w1; ++w) {
    co += __popc(bo[w]);
    cv += __popc(bv[w]);
  }
  int to, tv;
  int ro = block_excl_scan<1024>(co, &to, sh);
  int rv = block_excl_scan<1024>(cv, &tv, sh);
  uint32_t* pf = prefO + (size_t)g * (words + 1);
  int32_t* lo = cleanO + (size_t)g * cap_s;
  int32_t* lv = cleanV + (size_t)g * cap_v;
  for (int w = w0; w < w1; ++w) {
    pf[w] = (uint32_t)ro;
    uint32_t x = bo[w];
    while (x) {
      int bit = __ffs(x) - 1;
      x &= x - 1;
      if (ro < cap_s) lo[ro] = 32 * w + bit;
      ++ro;
    }
    x = bv[w];
    while (x) {
      int bit = __ffs(x) - 1;
      x &= x - 1;
      if (rv < cap_v) lv[rv] = 32 * w + bit;
      ++rv;
    }
  }
  if (tid == 0) {
    pf[words] = (uint32_t)to;
    counts[4 * g + 0] = min(to, cap_s);
    counts[4 * g + 1] = min(tv, cap_v);
  }
}

// per head: clusters of sorted offsets whose neighbours are at most `gap` apart
__global__ __launch_bounds__(1024) void ws_cluster_kernel(const int32_t* __restrict__ cleanO,
                                                          int cap_s, int gap, int32_t* clLo,
                                                          int32_t* clHi, int32_t* counts) {
  __shared__ int sh[17];
  const int g = blockIdx.x, tid = threadIdx.x;
  const int nO = counts[4 * g + 0];
  const int32_t* c = cleanO + (size_t)g * cap_s;
  const int per = (nO + 1023) / 1024;
  const int t0 = min(tid * per, nO), t1 = min(t0 + per, nO);
  int st = 0;
  for (int t = t0; t < t1; ++t) st += (t == 0 || c[t] - c[t - 1] > gap) ? 1 : 0;
  int tot;
  int id = block_excl_scan<1024>(st, &tot, sh) - 1;
  int32_t* lo = clLo + (size_t)g * cap_s;
  int32_t* hi = clHi + (size_t)g * cap_s;
  for (int t = t0; t < t1; ++t) {
    if (t == 0 || c[t] - c[t - 1] > gap) lo[++id] = c[t];
    if (t == nO - 1 || c[t + 1] - c[t] > gap) hi[id] = c[t];
  }
  if (tid == 0) counts[4 * g + 2] = tot;
}

// ---------------------------------------------------------------- attention

constexpr int kWaves = 8;               // waves per workgroup (two per SIMD)
constexpr int kThreads = kWaves * 64;

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int n, hkv, group, hpw, nsplit, nblocks, bmp;
  float c;  // scale * log2(e)
  const uint32_t* bitO;
  const uint32_t* bitV;
  int stride;
  const uint32_t* prefO;
  int words;
  const int32_t* cleanV;
  int cap_v;
  const int32_t* clLo;
  const int32_t* clHi;
  int cap_s;
  const int32_t* counts;
  unsigned long long* stats;
};

template <bool F32>
__device__ __forceinline__ u32x4 load8(const void* base, size_t elem) {
  if constexpr (F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    const float4 a = p[0], b = p[1];
    return u32x4{pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(b.x, b.y), pack_bf16(b.z, b.w)};
  } else {
    return *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem);
  }
}

// load through the scalar cache: the address must be wave-uniform and the
// memory must not change while the kernel runs
template <typename T>
__device__ __forceinline__ T ldc(const T* ptr, long idx) {
  return ((const __attribute__((address_space(4))) T*)ptr)[idx];
}

// Tile sequence of one workgroup: contiguous key tiles (code >= 0, the tile
// index) reached by the slash clusters in ascending key order, then tiles of
// gathered columns (code = -1 - chunk).  All state is wave-uniform.
struct TileSeq {
  const int32_t* clo;
  const int32_t* chi;
  int c, t, thi, next_t, i0, i1;
  int chunk, nchunks;
  bool dense;
};

// XOR swizzle of the 16-byte chunks of LDS row r, chosen so that both the
// MFMA operand reads of K (16 consecutive rows, one chunk) and the transposing
// reads of V (4 consecutive rows, two adjacent chunks) hit distinct banks
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

template <int D, bool F32>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p) {
  constexpr int KS = D / 16;            // k-steps of Q K^T
  constexpr int DT = D / 32;            // 32-row tiles of O^T
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int ROWB = D * 2;           // bytes per bf16 row
  constexpr int TILEB = kBN * ROWB;     // bytes per K (or V) tile
  constexpr int NST = 4;                // pipeline stages
  constexpr int RPD = 1024 / ROWB;      // rows per 1 KiB DMA (one wave, 16 B per lane)
  constexpr int NDMA = kBN / kWaves / RPD;  // DMAs per wave per matrix per tile
  static_assert(NDMA >= 1 && NDMA * RPD * kWaves == kBN, "tile split");
  // K stages at [0, NST*TILEB), V stages at [NST*TILEB, 2*NST*TILEB)
  __shared__ __align__(16) uint8_t kv_lds[2 * NST * TILEB];
  __shared__ __align__(16) int glist[kListCap];
  __shared__ int wcnt[kWaves + 1];
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8* const kv_base = (lds_u8*)kv_lds;

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, ql = lane & 31;
  const int wave = wave_uniform(tid >> 6);  // keep everything derived from it in SGPRs
  const int n = p.n;
  // block -> (KV head, head split, query block); consecutive blocks go to
  // different XCDs, so head g lands on XCD g and its K/V stays in that L2
  const int g = blockIdx.x % p.hkv;
  const int rest = blockIdx.x / p.hkv;
  const int split = rest % p.nsplit;
  const int b = p.nblocks - 1 - rest / p.nsplit;  // longest causal rows first
  const int i0 = b * p.bmp;
  const int i1 = min(i0 + p.bmp, n) - 1;
  const int head = g * p.group + split * p.hpw + (wave % p.hpw);
  const int i0w = i0 + 32 * (wave / p.hpw);
  const int qrow = i0w + ql;
  const bool wave_rows = i0w < n;
  const size_t kv_head = (size_t)g * n;

  const uint32_t* bo = p.bitO + (size_t)g * p.stride + kPrePad;
  const uint32_t* bv = p.bitV + (size_t)g * p.stride + kPrePad;
  const uint32_t* pfo = p.prefO + (size_t)g * (p.words + 1);
  // number of selected offsets below x (0 <= x <= n)
  auto prefix = [&](int x) -> int {
    const int w = x >> 5, sh = x & 31;
    return (int)ldc(pfo, w) + __popc(ldc(bo, w) & (sh ? ((1u << sh) - 1u) : 0u));
  };
  // does some offset link a row of this block to key tile T?
  auto tile_active = [&](int T) -> bool {
    const int wl = max(0, i0 - (T + 1) * kBN + 1), wh = i1 - T * kBN;
    return prefix(wh + 1) - prefix(wl) > 0;
  };
  // In a full block every tile of a cluster's key range is active; the last
  // block may be shorter than BMP rows, so there tiles are tested.
  const bool partial = i1 < i0 + p.bmp - 1;

  // Q^T fragments (B operand): lane holds row qrow, head dims 16s + 8*half .. +7
  bf16x8 qf[KS];
  {
    const size_t ro = ((size_t)head * n + min(qrow, n - 1)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 raw = load8<F32>(p.q, ro + 16 * s + 8 * half);
      if (qrow >= n) raw = u32x4{0u, 0u, 0u, 0u};
      qf[s] = as_bf16x8(raw);
    }
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;
  float m_run = kNoMax, l_run = 0.f;
  int n_dense = 0, n_gath = 0;

  // ---- tile sequence
  TileSeq seq;
  {
    seq.clo = p.clLo + (size_t)g * p.cap_s;
    seq.chi = p.clHi + (size_t)g * p.cap_s;
    const int ncl = ldc(p.counts, 4 * g + 2);
    int lo = 0, hi = ncl;  // first cluster whose smallest offset exceeds i1
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (ldc(seq.clo, mid) <= i1) lo = mid + 1;
      else hi = mid;
    }
    seq.c = lo - 1;
    seq.t = 1;
    seq.thi = 0;
    seq.next_t = 0;
    seq.i0 = i0;
    seq.i1 = i1;
    seq.chunk = 0;
    seq.nchunks = 0;
    seq.dense = true;
  }
  // next tile code, or INT_MIN when the sequence is exhausted
  auto next_tile = [&]() -> int {
    if (seq.dense) {
      while (true) {
        if (seq.t <= seq.thi) {
          const int t = seq.t++;
          if (partial && !tile_active(t)) continue;
          return t;
        }
        if (seq.c < 0) break;
        const int olo = ldc(seq.clo, seq.c), ohi = ldc(seq.chi, seq.c);
        --seq.c;
        const int klo = max(0, i0 - ohi), khi = i1 - olo;
        seq.t = max(klo / kBN, seq.next_t);
        seq.thi = khi / kBN;
        seq.next_t = max(seq.next_t, seq.thi + 1);
      }
      seq.dense = false;
    }
    if (seq.chunk < seq.nchunks) return -1 - seq.chunk++;
    return INT_MIN;
  };

  // ---- staging.  K and V tiles live row-major in LDS (bf16, chunk-swizzled)
  // and are filled by LDS-DMA buffer loads: each wave moves NDMA KiB of K and
  // of V per tile, lane l writing 16 bytes at the wave's base + 16 l.  The
  // buffer resources cover exactly this head's n rows, so rows at or past n
  // (the tail tile, gathered padding n, absent tiles) arrive as zeros.
  constexpr int GROWB = D * (F32 ? 4 : 2);  // bytes per row in HBM
  const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const char*>(p.k) + kv_head * GROWB), (short)0, n * GROWB, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const char*>(p.v) + kv_head * GROWB), (short)0, n * GROWB, kBufferFlags);
  const u32x4 wk = buffer_words(static_cast<const char*>(p.k) + kv_head * GROWB, (uint32_t)(n * GROWB));
  const u32x4 wv = buffer_words(static_cast<const char*>(p.v) + kv_head * GROWB, (uint32_t)(n * GROWB));
  int dma_row[NDMA], dma_chunk[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int r = wave * (kBN / kWaves) + i * RPD + lane / CH;
    dma_row[i] = r;
    dma_chunk[i] = (lane % CH) ^ swz<D>(r);  // the source chunk this lane's LDS slot holds
  }
  // fetch tile `code` into the stage at kdst / vdst (code INT_MIN: an absent
  // tile, all zeros)
  // The wait-count pass treats the DMA's address register as still in use
  // until the load lands, so letting the register allocator hand it to the
  // next LDS read costs a vmcnt(0) in the middle of the step.  Holding the
  // offsets live to the end of the step avoids that.
  unsigned dma_off[NDMA];
  auto stage_into = [&](int code, lds_u8* __restrict__ kdst, lds_u8* __restrict__ vdst) {
    const int* gk = glist + (code < 0 && code != INT_MIN ? (-1 - code) * kBN : 0);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int r = dma_row[i];
      const int gkey = gk[r];  // read unconditionally so no branch splits the step
      const int key = code >= 0 ? code * kBN + r : (code == INT_MIN ? n : gkey);
      const int kbase = (wave * (kBN / kWaves) + i * RPD) * ROWB;
      if constexpr (F32) {
        const unsigned off = (unsigned)key * GROWB + dma_chunk[i] * 32;
        const u32x4 k0 = __builtin_amdgcn_raw_buffer_load_b128(rsk, (int)off, 0, 0);
        const u32x4 k1 = __builtin_amdgcn_raw_buffer_load_b128(rsk, (int)(off + 16), 0, 0);
        const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(rsv, (int)off, 0, 0);
        const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(rsv, (int)(off + 16), 0, 0);
        auto cvt = [](const u32x4& a, const u32x4& c) {
          return u32x4{pack_bf16(__uint_as_float(a[0]), __uint_as_float(a[1])),
                       pack_bf16(__uint_as_float(a[2]), __uint_as_float(a[3])),
                       pack_bf16(__uint_as_float(c[0]), __uint_as_float(c[1])),
                       pack_bf16(__uint_as_float(c[2]), __uint_as_float(c[3]))};
        };
        *(__attribute__((address_space(3))) u32x4*)(kdst + kbase + 16 * lane) = cvt(k0, k1);
        *(__attribute__((address_space(3))) u32x4*)(vdst + kbase + 16 * lane) = cvt(v0, v1);
      } else {
        const unsigned off = (unsigned)key * GROWB + dma_chunk[i] * 16;
        dma16(wk, (uint32_t)(uintptr_t)(kdst + kbase), off);
        dma16(wv, (uint32_t)(uintptr_t)(vdst + kbase), off);
        dma_off[i] = off;
      }
    }
  };
  lds_u8* const k_region = kv_base;
  lds_u8* const v_region = kv_base + NST * TILEB;
  auto stage_tile = [&](int code, int st) { stage_into(code, k_region + st * TILEB, v_region + st * TILEB); };
  // Offset-bitmap words for a contiguous tile.  The wave's rows need offsets
  // [i0w - j0 - 63, i0w - j0 + 31], which lie in four consecutive words; they
  // come through the scalar cache and each lane picks its three.
  auto load_sw = [&](int code, uint32_t (&sw)[4]) {
    const int wq = code >= 0 ? (i0w - code * kBN - (kBN - 1)) >> 5 : 0;
    const int wc = max(wq, -kPrePad);
#pragma unroll
    for (int k = 0; k < 4; ++k) sw[k] = ldc(bo, wc + k);
  };
  // Per lane, a 64-bit word K with bit kk set when key kk of the tile is in
  // S_qrow.  The lane's scores are keys kk = 32*sk + 8*a + 4*half + bb (sk,
  // a, bb the element coordinates), so Kh = K >> (4*half) puts element
  // (sk, a, bb) at bit 8*a + bb of word sk.
  auto key_word = [&](int code, const uint32_t (&sw)[4], uint32_t& kh0, uint32_t& kh1) {
    uint32_t k0 = 0u, k1 = 0u;
    if (code >= 0) {
      const int j0 = code * kBN;
      const int dq = qrow - j0;  // largest causal key index of this row
      // bits of the offset bitmap from offset dq - 63 upward: bit x <-> key 63 - x
      const int base = i0w - j0 - (kBN - 1);
      const bool up = ((base & 31) + ql) >= 32;  // this lane's window starts one word on
      const uint32_t b0 = up ? sw[1] : sw[0], b1 = up ? sw[2] : sw[1], b2 = up ? sw[3] : sw[2];
      const int sh = (dq - (kBN - 1)) & 31;
      const uint32_t l0 = __builtin_amdgcn_alignbit(b1, b0, sh);
      const uint32_t l1 = __builtin_amdgcn_alignbit(b2, b1, sh);
      k0 = __builtin_bitreverse32(l1);
      k1 = __builtin_bitreverse32(l0);
      const uint32_t vw0 = ldc(bv, j0 >> 5), vw1 = ldc(bv, (j0 >> 5) + 1);
      // columns are visible up to key dq
      const uint32_t c0 = dq >= 31 ? ~0u : (dq < 0 ? 0u : ((2u << dq) - 1u));
      const uint32_t c1 = dq >= 63 ? ~0u : (dq < 32 ? 0u : ((2u << (dq - 32)) - 1u));
      k0 |= vw0 & c0;
      k1 |= vw1 & c1;
    } else if (code != INT_MIN) {
      // gathered keys ascend (padding n sorts last): the visible ones are a prefix
      const int* keys = &glist[(-1 - code) * kBN];
      int lo = 0;
#pragma unroll
      for (int step = 32; step > 0; step >>= 1)
        if (keys[lo + step - 1] <= qrow) lo += step;
      const int cnt = lo + (lo == 63 && keys[63] <= qrow ? 1 : 0);
      k0 = cnt >= 32 ? ~0u : ((1u << cnt) - 1u);
      k1 = cnt >= 64 ? ~0u : (cnt <= 32 ? 0u : ((1u << (cnt - 32)) - 1u));
    }
    kh0 = __builtin_amdgcn_alignbit(k1, k0, 4 * half);
    kh1 = k1 >> (4 * half);
  };

  // per-lane LDS byte offsets of the MFMA operand reads, for stage 0
  int koff[KS];  // K rows ql (+32 via the immediate), chunk 2*kk + half
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) koff[kk] = ql * ROWB + 16 * ((2 * kk + half) ^ swz<D>(ql));
  // V^T through ds_read_b64_tr_b16: in each 16-lane group, source lane
  // j = 4r + pp reads 4 values of row r at columns 4*pp.., and output lane
  // i = 4pp' + q receives column i of rows 0..3.  Group G16 = 2*h + dgrp
  // covers head dims 32*dt + 16*dgrp .. +15 and keys 4h..4h+3 (part 0) or
  // 8+4h.. (part 1) of each 16-key chunk: the slots the P^T operand uses.
  int voff[2][DT];
  {
    const int g16 = lane >> 4, j = lane & 15, rr = j >> 2, pp = j & 3, hh = g16 >> 1, dgrp = g16 & 1;
#pragma unroll
    for (int part = 0; part < 2; ++part)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int row = 8 * part + 4 * hh + rr;
        const int chunk = 4 * dt + 2 * dgrp + (pp >> 1);
        voff[part][dt] = row * ROWB + 16 * (chunk ^ swz<D>(row)) + 8 * (pp & 1);
      }
  }
  typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
  auto qk_part = [&](const lds_u8* kr, f32x16& s0, f32x16& s1, int k_lo, int k_hi) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (kk < k_lo || kk >= k_hi) continue;
      const bf16x8 a0 = *(const lds_bf16x8*)(kr + koff[kk]);
      const bf16x8 a1 = *(const lds_bf16x8*)(kr + koff[kk] + 32 * ROWB);
      s0 = mfma32(a0, qf[kk], s0);
      s1 = mfma32(a1, qf[kk], s1);
    }
  };
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  auto read_vt = [&](const lds_u8* vr, int part, int dt, int c4) -> v4i16 {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(vr + voff[part][dt] + c4 * 16 * ROWB));
  };
  // move the operand offsets one stage on (stage s -> s+1 mod NST)
  auto advance = [&](int (&o)[KS], int from) {
    const int delta = from == NST - 1 ? -(NST - 1) * TILEB : TILEB;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) o[kk] += delta;
  };
  auto advance_v = [&](int from) {
    const int delta = from == NST - 1 ? -(NST - 1) * TILEB : TILEB;
#pragma unroll
    for (int part = 0; part < 2; ++part)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) voff[part][dt] += delta;
  };
  constexpr int kWaitAfter = 2 * NDMA;  // DMAs issued per step after the awaited tile

  // ---- rounds: each gathers up to kListCap uncovered columns; the first
  //      round also walks the contiguous tiles
  const int32_t* cv = p.cleanV + (size_t)g * p.cap_v;
  int total_v;
  {
    const int nv = ldc(p.counts, 4 * g + 1);
    int lo = 0, hi = nv;  // columns <= i1
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (ldc(cv, mid) <= i1) lo = mid + 1;
      else hi = mid;
    }
    total_v = lo;
  }
  int cursor = 0;
  bool first_round = true;
  while (first_round || cursor < total_v) {
    // gather the next batch of columns whose tile no offset reaches
    int fill = 0;
    while (cursor < total_v && fill + kThreads <= kListCap) {
      const int idx = cursor + tid;
      bool keep = false;
      int col = 0;
      if (idx < total_v) {
        col = cv[idx];
        keep = !tile_active(col / kBN);
      }
      const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
      const int below_l = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      if (lane == 0) wcnt[wave] = __popcll(bal);
      __syncthreads();
      int before = 0, all = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int cw = wcnt[w];
        before += w < wave ? cw : 0;
        all += cw;
      }
      if (keep) glist[fill + before + below_l] = col;
      fill += all;
      cursor += kThreads;
      __syncthreads();
    }
    // pad the last gathered chunk with n: sorts after every key, reads as zeros
    for (int r = fill + tid; r < ((fill + kBN - 1) / kBN) * kBN; r += kThreads) glist[r] = n;
    seq.chunk = 0;
    seq.nchunks = (fill + kBN - 1) / kBN;
    if (!first_round) seq.dense = false;
    first_round = false;
    __syncthreads();

    // Software pipeline over the round's tiles, NST stages deep.  Tile t lives
    // in stage t % NST.  Step t: start the DMA of tile t+3, compute S(t+1) =
    // K(t+1) Q^T on the matrix cores alongside the softmax of tile t, add
    // V(t) P(t), then wait for this wave's share of tile t+2 and meet at the
    // barrier, after which tile t+2 is complete and stage (t-1) % NST is free.
    int cur = next_tile();
    if (cur == INT_MIN) continue;
    int nxt = next_tile();
    int n2 = nxt != INT_MIN ? next_tile() : INT_MIN;
    uint32_t sw_n[4], sw_nn[4];
    uint32_t kc0, kc1;
    f32x16 c0, c1;
    {
      uint32_t sw_c[4];
      load_sw(cur, sw_c);
      load_sw(nxt, sw_n);
      stage_tile(cur, 0);
      stage_tile(nxt, 1);
      stage_tile(n2, 2);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      key_word(cur, sw_c, kc0, kc1);
#pragma unroll
      for (int e = 0; e < 16; ++e) c0[e] = c1[e] = 0.f;
      qk_part(k_region, c0, c1, 0, KS);  // stage 0
    }
    advance(koff, 0);  // K operand reads now point at stage 1
    int t = 0;
    // One step.  The four LDS pointers never overlap in what they touch (K
    // and V of the stages being read, the stage being filled), which lets the
    // compiler keep the DMA in flight across the operand reads.
    auto step = [&](const lds_u8* __restrict__ krd, const lds_u8* __restrict__ vrd,
                    lds_u8* __restrict__ kdma, lds_u8* __restrict__ vdma, int n3) {
      // -- branchy part: key word of tile t+1, mask and row max of tile t, the
      //    rare rescale.  No K/V reads or DMA happen here.
      load_sw(n2, sw_nn);
      uint32_t kn0, kn1;
      key_word(nxt, sw_n, kn0, kn1);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int bpos = 8 * (e >> 2) + (e & 3);
        const uint32_t m0 = (uint32_t)__builtin_amdgcn_sbfe((int)kc0, bpos, 1);
        const uint32_t m1 = (uint32_t)__builtin_amdgcn_sbfe((int)kc1, bpos, 1);
        c0[e] = __uint_as_float((m0 & __float_as_uint(c0[e])) | (~m0 & 0xff800000u));
        c1[e] = __uint_as_float((m1 & __float_as_uint(c1[e])) | (~m1 & 0xff800000u));
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 16; ++e)
        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(c0[e], c1[e]));
      mx = half_max(mx);
      const float mt = mx * p.c;
      if (__builtin_amdgcn_ballot_w64(mt > m_run + kTau)) {
        const float mnew = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[dt][e] *= alpha;
        m_run = mnew;
      }
      // -- straight-line part: start the DMA of tile t+3, then S(t+1) on the
      //    matrix cores alongside exp/convert of tile t, then O += V(t) P(t)
      stage_into(n3, kdma, vdma);
      f32x16 sn0, sn1;
#pragma unroll
      for (int e = 0; e < 16; ++e) sn0[e] = sn1[e] = 0.f;
      qk_part(krd, sn0, sn1, 0, KS);
      const float nm = -m_run;
      uint32_t pk[16];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pk[e] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(c0[2 * e], p.c, nm)),
                          __builtin_amdgcn_exp2f(fmaf(c0[2 * e + 1], p.c, nm)));
        pk[8 + e] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(c1[2 * e], p.c, nm)),
                              __builtin_amdgcn_exp2f(fmaf(c1[2 * e + 1], p.c, nm)));
      }
      // row sum of the bf16 probabilities the PV product uses
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int e = 0; e < 16; ++e)
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e]), ones, l_run, false);
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const bf16x8 pf = as_bf16x8(u32x4{pk[4 * c4], pk[4 * c4 + 1], pk[4 * c4 + 2], pk[4 * c4 + 3]});
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const v4i16 lo4 = read_vt(vrd, 0, dt, c4), hi4 = read_vt(vrd, 1, dt, c4);
          const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[dt] = mfma32(av, pf, acc[dt]);
        }
      }
      if constexpr (!F32) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) asm volatile("" ::"v"(dma_off[i]));
      }
      c0 = sn0;
      c1 = sn1;
      kc0 = kn0;
      kc1 = kn1;
    };
    while (true) {
      const int n3 = n2 != INT_MIN ? next_tile() : INT_MIN;
      if (cur >= 0) ++n_dense;
      else ++n_gath;
      const int sdma = (t + 3) % NST;
      step(k_region, v_region, k_region + sdma * TILEB, v_region + sdma * TILEB, n3);
      if (nxt == INT_MIN) break;
      // this wave's share of tile t+2 has landed once at most the loads of
      // this step are outstanding; the barrier then completes tile t+2 for all
      if constexpr (F32) __builtin_amdgcn_s_waitcnt(0x0F70);
      else __builtin_amdgcn_s_waitcnt(0x0F70 | kWaitAfter);
      __syncthreads();
#pragma unroll
      for (int w = 0; w < 4; ++w) sw_n[w] = sw_nn[w];
      advance(koff, (t + 1) % NST);
      advance_v(t % NST);
      cur = nxt;
      nxt = n2;
      n2 = n3;
      ++t;
    }
    // drain: every outstanding DMA lands before the next round reuses stages
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    // rewind the operand offsets to stage 0
    {
      const int kst = (t + 1) % NST, vst = t % NST;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) koff[kk] -= kst * TILEB;
#pragma unroll
      for (int part = 0; part < 2; ++part)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) voff[part][dt] -= vst * TILEB;
    }
  }

  // ---------------- finish: normalise, write O and lse
  const float lt = half_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (wave_rows && qrow < n) {
    const size_t ro = ((size_t)head * n + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * dt + 8 * a + 4 * half;
        const float o0 = acc[dt][4 * a] * inv, o1 = acc[dt][4 * a + 1] * inv;
        const float o2 = acc[dt][4 * a + 2] * inv, o3 = acc[dt][4 * a + 3] * inv;
        if constexpr (F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + ro + d0) = float4{o0, o1, o2, o3};
        } else {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + ro + d0) =
              u32x2{pack_bf16(o0, o1), pack_bf16(o2, o3)};
        }
      }
    if (half == 0 && p.lse)
      p.lse[(size_t)head * n + qrow] = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -__builtin_inff();
  }
  if (tid == 0) {
    atomicAdd(&p.stats[0], (unsigned long long)n_dense);
    atomicAdd(&p.stats[1], (unsigned long long)n_gath);
  }
}

int heads_per_block(int group) { return group < kWaves ? group : kWaves; }

}  // namespace

int attn_query_rows_per_block(int group) {
  (void)group;
  return 32 * kWaves;
}

hipError_t launch_attn(const void* q, const void* k, const void* v, bool f32, int h_q, int h_kv,
                       int n, int d, float scale, const int32_t* v_idx, const int32_t* v_cnt,
                       int cap_v, const int32_t* s_off, const int32_t* s_cnt, int cap_s, void* out,
                       float* lse, void* ws, hipStream_t stream) {
  const AttnWsLayout L(h_kv, n, cap_v, cap_s);
  char* base = static_cast<char*>(ws);
  uint32_t* bitO = reinterpret_cast<uint32_t*>(base + L.off_bitO);
  uint32_t* bitV = reinterpret_cast<uint32_t*>(base + L.off_bitV);
  uint32_t* prefO = reinterpret_cast<uint32_t*>(base + L.off_prefO);
  int32_t* cleanO = reinterpret_cast<int32_t*>(base + L.off_cleanO);
  int32_t* cleanV = reinterpret_cast<int32_t*>(base + L.off_cleanV);
  int32_t* clLo = reinterpret_cast<int32_t*>(base + L.off_clLo);
  int32_t* clHi = reinterpret_cast<int32_t*>(base + L.off_clHi);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.off_counts);
  unsigned long long* stats = reinterpret_cast<unsigned long long*>(base + L.off_stats);

  const int group = h_q / h_kv;
  const int hpw = heads_per_block(group);   // query heads per workgroup
  const int nsplit = group / hpw;           // workgroups sharing one block of a group
  const int bmp = 32 * (kWaves / hpw);      // query positions per workgroup

  const size_t nwords = (size_t)h_kv * L.stride;
  hipLaunchKernelGGL(ws_clear_kernel, dim3((unsigned)std::min<size_t>((nwords + 255) / 256, 2048)),
                     dim3(256), 0, stream, bitO, bitV, nwords, stats);
  const int capm = std::max(cap_v, cap_s);
  hipLaunchKernelGGL(ws_setbits_kernel, dim3((unsigned)((capm + 255) / 256), (unsigned)h_kv),
                     dim3(256), 0, stream, v_idx, v_cnt, cap_v, s_off, s_cnt, cap_s, n, bitO, bitV,
                     L.stride);
  hipLaunchKernelGGL(ws_scan_kernel, dim3((unsigned)h_kv), dim3(1024), 0, stream, bitO, bitV,
                     L.stride, L.words, prefO, cleanO, cap_s, cleanV, cap_v, counts);
  // offsets closer than bmp + 64 reach one contiguous run of 64-key tiles
  hipLaunchKernelGGL(ws_cluster_kernel, dim3((unsigned)h_kv), dim3(1024), 0, stream, cleanO,
                     cap_s, bmp + kBN - 1, clLo, clHi, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  AttnParams prm;
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.out = out;
  prm.lse = lse;
  prm.n = n;
  prm.hkv = h_kv;
  prm.group = group;
  prm.hpw = hpw;
  prm.nsplit = nsplit;
  prm.bmp = bmp;
  prm.nblocks = (n + bmp - 1) / bmp;
  prm.c = scale * kLog2e;
  prm.bitO = bitO;
  prm.bitV = bitV;
  prm.stride = L.stride;
  prm.prefO = prefO;
  prm.words = L.words;
  prm.cleanV = cleanV;
  prm.cap_v = cap_v;
  prm.clLo = clLo;
  prm.clHi = clHi;
  prm.cap_s = cap_s;
  prm.counts = counts;
  prm.stats = stats;
  const dim3 grid((unsigned)((long long)prm.nblocks * h_kv * nsplit));
  if (d == 128) {
    if (f32) hipLaunchKernelGGL((attn_kernel<128, true>), grid, dim3(kThreads), 0, stream, prm);
    else hipLaunchKernelGGL((attn_kernel<128, false>), grid, dim3(kThreads), 0, stream, prm);
  } else {
    if (f32) hipLaunchKernelGGL((attn_kernel<64, true>), grid, dim3(kThreads), 0, stream, prm);
    else hipLaunchKernelGGL((attn_kernel<64, false>), grid, dim3(kThreads), 0, stream, prm);
  }
  return hipGetLastError();
}

}  // namespace vs
