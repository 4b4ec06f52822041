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

template <int D, bool F32>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p) {
  constexpr int KS = D / 16;     // k-steps of Q K^T
  constexpr int DT = D / 32;     // 32-row tiles of O^T
  constexpr int KROW = D + 8;    // padded LDS row of K (bf16 elements)
  constexpr int VROW = kBN + 8;  // padded LDS row of V^T
  constexpr int KCH = D / 8;     // 16-byte chunks per K row
  __shared__ __align__(16) uint16_t k_lds[2][kBN * KROW];
  __shared__ __align__(16) uint16_t vt_lds[2][D * VROW];
  __shared__ __align__(16) int glist[kListCap];
  __shared__ int wcnt[kWaves + 1];

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

  // ---- staging: waves 0-3 stage V^T (transposed, key-permuted), waves 4-7 stage K.
  // K and V rows are read through buffer resources that cover exactly this
  // head's n rows: rows at or past n (the tail tile, gathered padding) read
  // as zeros with no branch.
  constexpr int ESZ = F32 ? 4 : 2;
  constexpr int ROWB = D * ESZ;  // bytes per K/V row
  const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const char*>(p.k) + kv_head * ROWB), (short)0, n * ROWB, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const char*>(p.v) + kv_head * ROWB), (short)0, n * ROWB, kBufferFlags);
  auto bload8 = [&](const __amdgpu_buffer_rsrc_t& rs, unsigned off) -> u32x4 {
    if constexpr (F32) {
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
      const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + 16), 0, 0);
      return u32x4{pack_bf16(__uint_as_float(a[0]), __uint_as_float(a[1])),
                   pack_bf16(__uint_as_float(a[2]), __uint_as_float(a[3])),
                   pack_bf16(__uint_as_float(c[0]), __uint_as_float(c[1])),
                   pack_bf16(__uint_as_float(c[2]), __uint_as_float(c[3]))};
    } else {
      return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
    }
  };
  constexpr int KRS = kThreads / 2 / KCH;  // K rows staged per pass of 256 threads
  const int k_row0 = (tid - 256) / KCH, k_c8 = (tid - 256) % KCH;
  const int v_kgp = tid & 15, v_dc = tid >> 4;
  u32x4 pre[4];
  // global -> registers: waves 4-7 fetch K of tile ck, waves 0-3 fetch V of tile cv
  auto load_kv = [&](int ck, int cv) {
    if (wave >= 4) {
      if (ck != INT_MIN) {
        const int* gk = glist + (ck < 0 ? (-1 - ck) * kBN : 0);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          if (it * KRS < kBN) {
            const int r = k_row0 + KRS * it;
            const int key = ck >= 0 ? ck * kBN + r : gk[r];
            pre[it] = bload8(rsk, (unsigned)key * ROWB + k_c8 * 8 * ESZ);
          }
        }
      }
    } else if (cv != INT_MIN && v_dc < D / 8) {
      int4 keys4;
      if (cv >= 0) {
        const int k0 = cv * kBN + 4 * v_kgp;
        keys4 = int4{k0, k0 + 1, k0 + 2, k0 + 3};
      } else {
        keys4 = *reinterpret_cast<const int4*>(&glist[(-1 - cv) * kBN + 4 * v_kgp]);
      }
      pre[0] = bload8(rsv, (unsigned)keys4.x * ROWB + v_dc * 8 * ESZ);
      pre[1] = bload8(rsv, (unsigned)keys4.y * ROWB + v_dc * 8 * ESZ);
      pre[2] = bload8(rsv, (unsigned)keys4.z * ROWB + v_dc * 8 * ESZ);
      pre[3] = bload8(rsv, (unsigned)keys4.w * ROWB + v_dc * 8 * ESZ);
    }
  };
  // registers -> LDS: K into k_lds[kb] (when has_k), V^T into vt_lds[vb] (when has_v)
  auto store_kv = [&](int kb, bool has_k, int vb, bool has_v) {
    if (wave >= 4) {
      if (has_k) {
#pragma unroll
        for (int it = 0; it < 4; ++it)
          if (it * KRS < kBN)
            *reinterpret_cast<u32x4*>(&k_lds[kb][(k_row0 + KRS * it) * KROW + 8 * k_c8]) = pre[it];
      }
    } else if (has_v && v_dc < D / 8) {
      // slot of these 4 keys inside their 16-key chunk: the order in which
      // the two wave halves consume keys as the k index of O^T += V^T P^T
      const int pos = 16 * (v_kgp >> 2) + 8 * (v_kgp & 1) + 4 * ((v_kgp >> 1) & 1);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int w = dd >> 1;
        const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(pre[1][w], pre[0][w], sel);
        const uint32_t hi = __builtin_amdgcn_perm(pre[3][w], pre[2][w], sel);
        *reinterpret_cast<u32x2*>(&vt_lds[vb][(8 * v_dc + dd) * VROW + pos]) = u32x2{lo, hi};
      }
    }
  };
  // offset-bitmap words this lane's row needs for a contiguous tile:
  // offsets qrow - j for the tile's keys are [qrow - j0 - 63, qrow - j0]
  auto load_bw = [&](int code, uint32_t (&bw)[3]) {
    if (code >= 0) {
      const int wq = max((qrow - code * kBN - (kBN - 1)) >> 5, -kPrePad);
      bw[0] = bo[wq];
      bw[1] = bo[wq + 1];
      bw[2] = bo[wq + 2];
    }
  };
  // Per lane, a 64-bit word K with bit kk set when key kk of the tile is in
  // S_qrow.  The lane's scores are keys kk = 32*sk + 8*a + 4*half + bb (sk,
  // a, bb the element coordinates), so Kh = K >> (4*half) puts element
  // (sk, a, bb) at bit 8*a + bb of word sk.
  auto key_word = [&](int code, const uint32_t (&bw)[3], uint32_t& kh0, uint32_t& kh1) {
    uint32_t k0 = 0u, k1 = 0u;
    if (code >= 0) {
      const int j0 = code * kBN;
      const int dq = qrow - j0;  // largest causal key index of this row
      // bits of the offset bitmap from offset dq - 63 upward: bit x <-> key 63 - x
      const int sh = (dq - (kBN - 1)) & 31;
      const uint32_t l0 = __builtin_amdgcn_alignbit(bw[1], bw[0], sh);
      const uint32_t l1 = __builtin_amdgcn_alignbit(bw[2], bw[1], sh);
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
      // lo keys are <= qrow (0..63); one more probe decides 64
      const int cnt = lo + (lo == 63 && keys[63] <= qrow ? 1 : 0);
      k0 = cnt >= 32 ? ~0u : ((1u << cnt) - 1u);
      k1 = cnt >= 64 ? ~0u : (cnt <= 32 ? 0u : ((1u << (cnt - 32)) - 1u));
    }
    kh0 = __builtin_amdgcn_alignbit(k1, k0, 4 * half);
    kh1 = k1 >> (4 * half);
  };
  // S^T of this wave's rows against the 64 keys in k_lds[kb], k-steps [k_lo, k_hi)
  auto qk_part = [&](int kb, f32x16& s0, f32x16& s1, int k_lo, int k_hi) {
    const uint16_t* kp = k_lds[kb];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (kk < k_lo || kk >= k_hi) continue;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&kp[ql * KROW + 16 * kk + 8 * half]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&kp[(32 + ql) * KROW + 16 * kk + 8 * half]);
      s0 = mfma32(a0, qf[kk], s0);
      s1 = mfma32(a1, qf[kk], s1);
    }
  };

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

    // Software pipeline over the round's tiles.  In step t the matrix cores
    // compute S(t+1) = K(t+1) Q^T while the vector units run the softmax of
    // tile t, then O += V(t) P(t).  K is staged two tiles ahead and V one,
    // so two LDS buffers of each suffice with one barrier per step.
    int cur = next_tile();
    if (cur == INT_MIN) continue;
    int nxt = next_tile();
    uint32_t bw_n[3] = {0u, 0u, 0u}, bw_nn[3] = {0u, 0u, 0u};
    {
      uint32_t bw_c[3] = {0u, 0u, 0u};
      load_bw(cur, bw_c);
      load_bw(nxt, bw_n);
      load_kv(cur, cur);
      store_kv(0, true, 0, true);
      if (nxt != INT_MIN) {
        load_kv(nxt, INT_MIN);
        store_kv(1, true, 0, false);
      }
      __syncthreads();
      uint32_t kc0, kc1;
      key_word(cur, bw_c, kc0, kc1);
      f32x16 c0, c1;
#pragma unroll
      for (int e = 0; e < 16; ++e) c0[e] = c1[e] = 0.f;
      qk_part(0, c0, c1, 0, KS);
      int t = 0;
      while (true) {
        const int nn = nxt != INT_MIN ? next_tile() : INT_MIN;
        load_kv(nn, nxt);
        load_bw(nn, bw_nn);
        uint32_t kn0, kn1;
        key_word(nxt, bw_n, kn0, kn1);
        if (cur >= 0) ++n_dense;
        else ++n_gath;
        const int kbn = (t + 1) & 1, vbc = t & 1;
        f32x16 sn0, sn1;
#pragma unroll
        for (int e = 0; e < 16; ++e) sn0[e] = sn1[e] = 0.f;

        // -- softmax of tile t, with the first half of S(t+1) in flight
        qk_part(kbn, sn0, sn1, 0, KS / 2);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int b = 8 * (e >> 2) + (e & 3);
          const uint32_t m0 = (uint32_t)__builtin_amdgcn_sbfe((int)kc0, b, 1);
          const uint32_t m1 = (uint32_t)__builtin_amdgcn_sbfe((int)kc1, b, 1);
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
        qk_part(kbn, sn0, sn1, KS / 2, KS);
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
        // -- O^T += V^T(t) P^T(t)
        const uint16_t* vp = vt_lds[vbc];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const bf16x8 pf = as_bf16x8(u32x4{pk[4 * c4], pk[4 * c4 + 1], pk[4 * c4 + 2], pk[4 * c4 + 3]});
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const bf16x8 av = *reinterpret_cast<const bf16x8*>(&vp[(32 * dt + ql) * VROW + 16 * c4 + 8 * half]);
            acc[dt] = mfma32(av, pf, acc[dt]);
          }
        }
        if (nxt == INT_MIN) break;
        store_kv(t & 1, nn != INT_MIN, (t + 1) & 1, true);
        __syncthreads();
        c0 = sn0;
        c1 = sn1;
        kc0 = kn0;
        kc1 = kn1;
#pragma unroll
        for (int w = 0; w < 3; ++w) bw_n[w] = bw_nn[w];
        cur = nxt;
        nxt = nn;
        ++t;
      }
    }
    __syncthreads();
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
