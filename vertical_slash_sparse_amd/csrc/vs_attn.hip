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
//    of the per-cluster ranges, no n x n structure).  Tiles inside a
//    gap-free cluster hold only selected pairs for every row of the block
//    and run first without masks; every other tile is masked per element by
//    (j <= i) and (offset bit or column bit), from a 64-bit key word per lane
//    built out of wave-uniform bitmap windows (a bit extract and a bitwise
//    select per element).  Columns that no processed tile covers are then
//    gathered 64 at a time into tiles of their own (unmasked when they all
//    lie below the block).
//  * Math per 64-key tile and 32 query rows: S^T = K Q^T on
//    v_mfma_f32_32x32x16_bf16 (K from LDS, Q^T held in registers), online
//    softmax in fp32 on the transposed scores (each lane owns one query row,
//    so row statistics need one cross-half exchange), P^T reused directly as
//    the B operand of O^T += V^T P^T with V^T staged in LDS in a matching
//    key order.  Probabilities are taken against the running maximum, which
//    only moves when some p of a tile could exceed 2^8 (the result is
//    unchanged; p stays at most 2^8 in fp32/bf16); a lane's sum of its p,
//    needed anyway, bounds each of them, so the tile's own maximum is
//    computed only when that sum is over 2^8.
#include <algorithm>
#include <atomic>
#include <cfloat>
#include <climits>

#include <type_traits>
#include <vector>

#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

namespace {

// lazy rescale: the largest p (2^8, so 8 in log2 units above the running
// maximum) a tile may reach before the maximum is moved; 2^16 measured the
// same, as the maximum rarely moves after a row's first tile
constexpr float kPMax = 256.0f;
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
  if (blockIdx.x == 0 && threadIdx.x < kStatWords) stats[threadIdx.x] = 0ull;
}

// A packed batch's rows: sequence r / sets has lens[r / sets] positions, and
// only the words its tiles can read are cleared (pads, then its bitmap).
__global__ void ws_clear_rows_kernel(uint32_t* bitO, uint32_t* bitV, int stride,
                                     const int* __restrict__ lens, int sets,
                                     unsigned long long* stats) {
  const int r = blockIdx.x;
  const int nw = min(kPrePad + (lens[r / sets] + 31) / 32 + kPostPad, stride);
  for (int w = threadIdx.x; w < nw; w += blockDim.x) {
    bitO[(size_t)r * stride + w] = 0u;
    bitV[(size_t)r * stride + w] = 0u;
  }
  if (r == 0 && threadIdx.x < kStatWords) stats[threadIdx.x] = 0ull;
}

// lens (packed batch) null: every row covers positions [0, n)
__global__ void ws_setbits_kernel(const int32_t* __restrict__ v_idx, const int32_t* __restrict__ v_cnt,
                                  int cap_v, const int32_t* __restrict__ s_off,
                                  const int32_t* __restrict__ s_cnt, int cap_s, int n,
                                  const int* __restrict__ lens, int sets,
                                  uint32_t* bitO, uint32_t* bitV, int stride) {
  const int g = blockIdx.x;
  if (lens) n = lens[g / sets];
  const int cv = min(max(v_cnt[g], 0), cap_v);
  const int cs = min(max(s_cnt[g], 0), cap_s);
  const int step = gridDim.y * blockDim.x;
  for (int t = blockIdx.y * blockDim.x + threadIdx.x; t < max(cv, cs); t += step) {
    if (t < cv) {
      int x = v_idx[(size_t)g * cap_v + t];
      if (x >= 0 && x < n) atomicOr(&bitV[(size_t)g * stride + kPrePad + (x >> 5)], 1u << (x & 31));
    }
    if (t < cs) {
      int x = s_off[(size_t)g * cap_s + t];
      if (x >= 0 && x < n) atomicOr(&bitO[(size_t)g * stride + kPrePad + (x >> 5)], 1u << (x & 31));
    }
  }
}

// per head: prefix counts of the offset bitmap and sorted unique lists
__global__ __launch_bounds__(1024) void ws_scan_kernel(const uint32_t* __restrict__ bitO,
                                                       const uint32_t* __restrict__ bitV,
                                                       int stride, int words, uint32_t* prefO,
                                                       int32_t* cleanO, int cap_s,
                                                       int32_t* cleanV, int cap_v,
                                                       int32_t* counts,
                                                       const int* __restrict__ lens, int sets) {
  __shared__ int sh[17];
  const int g = blockIdx.x, tid = threadIdx.x;
  const size_t prow = (size_t)g * (words + 1);  // this row's prefix counts
  if (lens) words = (lens[g / sets] + 31) / 32;
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
  uint32_t* pf = prefO + prow;
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
constexpr int kRotRows = 32;            // blocks per XCD between head rotations
constexpr int kMasked = 0, kTested = 1, kNoMask = 2;  // softmax masking modes (see softmax)
constexpr int kThreads = kWaves * 64;
constexpr int kQueues = 8;  // item classes: one per XCD

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int n, hkv, group, hpw, nsplit, nblocks, bmp;
  // scale * log2(e) carried as a positive multiplier |c| and a sign: the sign
  // of c is folded into Q as it is loaded (every Q element flips), so that
  // the softmax sees scale * q.k through |c|, a free operand modifier.  A
  // zero scale is carried as the smallest normal float: every score then
  // rounds to 0 in the exponent, which is what a zero scale means.
  float c;
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
  const uint32_t* blk;  // block mode: key-block bitmap per (KV head, query block of 64)
  int blk_wpr;          // its words per row
  // Addressing.  Index sets belong to "set heads" g (a KV head, or a query
  // head when every query head has its own sets); set head g reads K/V head
  // g / kvdiv.  Row r of a head's sequence lives at row hstride * head +
  // row0 + r of the [heads][rows][d] tensors (hstride = n, row0 = 0 for one
  // sequence; a packed batch of sequences passes its total length and the
  // sequence's first row).
  int kvdiv;
  long long hstride;
  long long row0;
  // A packed batch in one launch (seq_tab null otherwise): the sequences in
  // workgroup order (longest first) as five int arrays of nseq + 1 entries,
  // seq_tab[0..]: first workgroup of each (then the grid size), [1]: its
  // length, [2]: its first row, [3]: its index s in the caller's lists, whose
  // set heads use workspace rows s * hkv .. s * hkv + hkv - 1.
  const int* seq_tab;
  int nseq;
  // Work items (one per 64-position block of a set head and head split, in
  // the order the mapping below gives) and their queues: workgroup w starts
  // with item w, then claims items of its class w % 8 (the XCD it runs on
  // when workgroups are dealt round-robin) from queue[w % 8], and once its
  // class is exhausted, items of the other classes.
  int nitems;
  unsigned* queue;  // kQueues counters, zero at launch
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
// the same at a 32-bit byte offset, which the load takes as a register offset
template <typename T>
__device__ __forceinline__ T ldc_at(const T* ptr, unsigned byte_off) {
  return *(const __attribute__((address_space(4))) T*)((const __attribute__((address_space(4))) char*)ptr + byte_off);
}

// XOR swizzle of the 16-byte chunks of LDS row r, chosen so that both the
// MFMA operand reads of K (16 consecutive rows, one chunk: the swizzles of
// any 16 aligned rows are distinct) and the transposing reads of V (two
// 16-lane groups together: 4 aligned rows, four adjacent chunks 4c .. 4c+3)
// hit distinct banks.  At d = 128 a row is 16 chunks: the row's low two bits
// pick the block of four chunks and the next two bits the chunk within it.
// At d = 64 a row is 8 chunks and two rows share a 256-byte bank window, so
// the bits above the row's parity do the same within each half.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Scheduling groups for the matrix half: npv products whose operand takes
// two LDS reads, then nqk taking one; each product's reads are issued
// `ahead` products before it.
template <int NPV, int NQK, int AHEAD>
struct MhalfOrder {
  static constexpr int reads(int i) { return i < NPV ? 2 : (i < NPV + NQK ? 1 : 0); }
  static constexpr int prologue_reads() {
    int r = 0;
    for (int i = 0; i < AHEAD; ++i) r += reads(i);
    return r;
  }
  template <int I>
  static __device__ __forceinline__ void emit() {
    if constexpr (I < NPV + NQK) {
      constexpr int r = reads(I + AHEAD);
      if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x080, r, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      emit<I + 1>();
    }
  }
};

// FULL: test each tile for "every key in every row's set" and skip the
// per-element masks there.  Worth it only when most tiles are full (the block
// mode's interior tiles, every offset selected): a set that leaves a few keys
// out of most tiles pays for the test and loses the interleaving of masks
// and maxima (measured 3.5 % slower on a 98 %-dense 256K layer).
template <int D, bool F32, bool BLK, bool FULL>
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
  // four spare entries: the pipelines read the code of step t+4 without a clamp
  __shared__ __align__(16) int glist[kListCap + 4];
  __shared__ int wcnt[kWaves + 1];
  // per cluster of one batch while a window of the tile list is written: its
  // first slot in the window, and its tiles as ranges [a, a + b) then c ..
  __shared__ int cl_pos[kThreads], cl_a[kThreads], cl_b[kThreads], cl_c[kThreads];
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8* const kv_base = (lds_u8*)kv_lds;

  __shared__ int next_item;

  // ---- persistent loop over work items.  The claim of the next item is
  // issued as an item starts and read when it ends, so its latency stays
  // hidden; only when a class runs dry does the search wait on atomics.
  const int cls = blockIdx.x % kQueues;
  const int nwg = gridDim.x;
  // item k of class c past the ones the grid starts with
  auto class_item = [&](int c, unsigned k) -> long long {
    const long long first = c < nwg ? (nwg - c + kQueues - 1) / kQueues : 0;
    return c + (long long)kQueues * (first + k);
  };
  for (int item = blockIdx.x; item < p.nitems;) {
    // lane-dependent values are formed afresh per item: hoisted out of the
    // loop they would stay live through every pipeline
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o, lane = tid & 63, half = lane >> 5, ql = lane & 31;
    const int wave = wave_uniform(tid >> 6);  // keep everything derived from it in SGPRs
    unsigned claim = 0;
    if (tid == 0) claim = atomicAdd(&p.queue[cls], 1u);
    int n = p.n, nblocks = p.nblocks, bid = item, wrow0 = 0;
    long long row0 = p.row0;
    if (p.seq_tab) {  // the sequence of this workgroup: the last one starting at or before it
      const int* tw = p.seq_tab;
      int lo = 0, hi = p.nseq - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ldc(tw, mid) <= bid) lo = mid;
        else hi = mid - 1;
      }
      const int stride = p.nseq + 1;
      bid -= ldc(tw, lo);
      n = ldc(tw, stride + lo);
      row0 = ldc(tw, 2 * stride + lo);
      wrow0 = ldc(tw, 3 * stride + lo) * p.hkv;
      nblocks = (n + p.bmp - 1) / p.bmp;
    }
    // block -> (KV head, head split, query block).  Consecutive blocks go to
    // different XCDs, so the workgroups an XCD runs at one time serve one head
    // and share its K/V in that XCD's L2.  Heads can differ in work (their sets
    // differ), so the head an XCD serves moves on every kRotRows of its blocks:
    // each XCD then takes a slice of every head and they finish together.
    const int rest = bid / p.hkv;
    const int g = (bid % p.hkv + rest / kRotRows) % p.hkv;
    const int wr = wrow0 + g;  // the workspace row of set head g's index sets
    const int split = rest % p.nsplit;
    const int b = nblocks - 1 - rest / p.nsplit;  // longest causal rows first
    const int i0 = b * p.bmp;
    const int i1 = min(i0 + p.bmp, n) - 1;
    const int head = g * p.group + split * p.hpw + (wave % p.hpw);
    const int i0w = i0 + 32 * (wave / p.hpw);
    const int qrow = i0w + ql;
    const bool wave_rows = i0w < n;
    const size_t hstride = (size_t)p.hstride;
    const float cpos = fabsf(p.c);  // the softmax multiplier (an operand modifier)
    const size_t kv_head = (size_t)(g / p.kvdiv) * hstride + row0;  // first K/V row of the sequence

    const uint32_t* bo = p.bitO + (size_t)wr * p.stride + kPrePad;
    const uint32_t* bv = p.bitV + (size_t)wr * p.stride + kPrePad;
    const uint32_t* pfo = p.prefO + (size_t)wr * (p.words + 1);
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

    // Q^T fragments (B operand): lane holds row qrow, head dims 16s + 8*half .. +7.
    // Loaded when the first pipeline starts, together with its first K/V tiles:
    // loads complete in order, so Q loaded up front would be waited for by the
    // tile-list build's own loads, and a block with no tiles never needs it.
    bf16x8 qf[KS];
    bool q_ready = false;
    auto load_q = [&]() {
      if (q_ready) return;
      q_ready = true;
      const size_t ro = ((size_t)head * hstride + row0 + min(qrow, n - 1)) * D;
      // a negative scale flips the sign of Q; the mask is formed here, not
      // ahead of time (the empty asm keeps the compiler from hoisting it into a
      // register held across the kernel)
      uint32_t cbits = __float_as_uint(p.c);
      asm volatile("" : "+s"(cbits));
      const uint32_t qx = (cbits >> 31) * 0x80008000u;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u32x4 raw = load8<F32>(p.q, ro + 16 * s + 8 * half);
#pragma unroll
        for (int e = 0; e < 4; ++e) raw[e] ^= qx;
        if (qrow >= n) raw = u32x4{0u, 0u, 0u, 0u};
        qf[s] = as_bf16x8(raw);
      }
    };

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;
    float m_run = kNoMax, l_run = 0.f;
    int n_dense = 0, n_gath = 0;

    // ---- LDS staging.  K and V tiles live row-major in LDS (bf16,
    // chunk-swizzled) in two rings of NST stages.  bf16 tiles arrive by LDS-DMA
    // buffer loads: each wave moves NDMA KiB of a tile, lane l writing 16 bytes
    // at the wave's base + 16 l.  The buffer resources cover exactly this
    // head's n rows, so rows at or past n (the tail tile, padding keys n, the
    // tiles past the end of a list) arrive as zeros.  fp32 tiles go through
    // registers and are rounded to bf16 on the way.
    constexpr int GROWB = D * (F32 ? 4 : 2);     // bytes per row in HBM
    constexpr int KREG = 0, VREG = NST * TILEB;  // ring offsets within kv_lds
    const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const char*>(p.k) + kv_head * GROWB), (short)0, n * GROWB, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const char*>(p.v) + kv_head * GROWB), (short)0, n * GROWB, kBufferFlags);
    const u32x4 wk = buffer_words(static_cast<const char*>(p.k) + kv_head * GROWB, (uint32_t)(n * GROWB));
    const u32x4 wv = buffer_words(static_cast<const char*>(p.v) + kv_head * GROWB, (uint32_t)(n * GROWB));
    int dma_row[NDMA], dma_col[NDMA];  // tile row and byte offset within the row this lane moves
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int r = wave * (kBN / kWaves) + i * RPD + lane / CH;
      dma_row[i] = r;
      dma_col[i] = ((lane % CH) ^ swz<D>(r)) * (F32 ? 32 : 16);  // the source chunk of this LDS slot
    }
    // The wait-count pass treats a DMA's address register as in use until the
    // load lands, so letting the register allocator hand it to a later LDS read
    // costs a vmcnt(0) in the middle of a step.  The offsets are held live to
    // the end of each V half instead.
    unsigned dma_off[2][NDMA];
    // fetch matrix `which` (0 K, 1 V) of the keys key[i] (one per DMA slot)
    // into LDS at byte `dst` of kv_lds
    auto stage_keys = [&](int which, const int (&key)[NDMA], int dst) {
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int kbase = dst + (wave * (kBN / kWaves) + i * RPD) * ROWB;
        const unsigned off = (unsigned)key[i] * GROWB + dma_col[i];
        if constexpr (F32) {
          const __amdgpu_buffer_rsrc_t rs = which ? rsv : rsk;
          const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
          const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + 16), 0, 0);
          *(__attribute__((address_space(3))) u32x4*)(kv_base + kbase + 16 * lane) =
              u32x4{pack_bf16(__uint_as_float(a[0]), __uint_as_float(a[1])),
                    pack_bf16(__uint_as_float(a[2]), __uint_as_float(a[3])),
                    pack_bf16(__uint_as_float(c[0]), __uint_as_float(c[1])),
                    pack_bf16(__uint_as_float(c[2]), __uint_as_float(c[3]))};
        } else {
          dma16(which ? wv : wk, (uint32_t)(uintptr_t)(kv_base + kbase), off);
          dma_off[which][i] = off;
        }
      }
    };
    // contiguous tile `code` (keys code*64 ..): the lane's offset within a
    // tile is fixed, so only the tile's wave-uniform base changes per call
    unsigned dma_lane[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) dma_lane[i] = (unsigned)dma_row[i] * GROWB + dma_col[i];
    auto stage_tile = [&](int which, int code, int dst) {
      if constexpr (BLK) {  // block mode measured 2 % faster with per-lane keys
        int key[NDMA];
#pragma unroll
        for (int i = 0; i < NDMA; ++i) key[i] = code * kBN + dma_row[i];
        stage_keys(which, key, dst);
        return;
      }
      const unsigned tb = (unsigned)__builtin_amdgcn_readfirstlane(code) * (unsigned)(kBN * GROWB);
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int kbase = dst + (wave * (kBN / kWaves) + i * RPD) * ROWB;
        const unsigned off = tb + dma_lane[i];
        if constexpr (F32) {
          const __amdgpu_buffer_rsrc_t rs = which ? rsv : rsk;
          const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
          const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + 16), 0, 0);
          *(__attribute__((address_space(3))) u32x4*)(kv_base + kbase + 16 * lane) =
              u32x4{pack_bf16(__uint_as_float(a[0]), __uint_as_float(a[1])),
                    pack_bf16(__uint_as_float(a[2]), __uint_as_float(a[3])),
                    pack_bf16(__uint_as_float(c[0]), __uint_as_float(c[1])),
                    pack_bf16(__uint_as_float(c[2]), __uint_as_float(c[3]))};
        } else {
          dma16(which ? wv : wk, (uint32_t)(uintptr_t)(kv_base + kbase), off);
          dma_off[which][i] = off;
        }
      }
    };

    // ---- key words.  Per lane, a 64-bit word K with bit kk set when key kk
    // of the tile is in S_qrow.  The lane's scores are keys kk = 32*sk + 8*a +
    // 4*half + bb (sk, a, bb the element coordinates), so Kh = K >> (4*half)
    // puts element (sk, a, bb) at bit 8*a + bb of word sk.
    struct BitWords {
      uint32_t o[4];  // offset-bitmap words covering the wave's windows
      uint32_t v[2];  // column-bitmap words of the tile's keys
    };
    // scalar loads for contiguous tile `code`: the wave's rows need offsets
    // [i0w - j0 - 63, i0w - j0 + 31], which lie in four consecutive words
    auto load_words = [&](int code, BitWords& w) {
      const int j0 = __builtin_amdgcn_readfirstlane(code) * kBN;
      const int wq = (i0w - j0 - (kBN - 1)) >> 5;
      // word index counted from the start of the zero pre-pad (further
      // below, the window holds only zeros), as a 32-bit byte offset
      const unsigned wc = (unsigned)__builtin_amdgcn_readfirstlane((max(wq, -kPrePad) + kPrePad) * 4);
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x4 o = ldc_at(reinterpret_cast<const u32x4*>(bo - kPrePad), wc);
      const u32x2 v = ldc_at(reinterpret_cast<const u32x2*>(bv), (unsigned)j0 >> 3);
#pragma unroll
      for (int k = 0; k < 4; ++k) w.o[k] = o[k];
      w.v[0] = v[0];
      w.v[1] = v[1];
    };
    auto key_word_tile = [&](int code, const BitWords& w, uint32_t& kh0, uint32_t& kh1) {
      const int j0 = code * kBN;
      const int dq = qrow - j0;  // largest causal key index of this row
      // bits of the offset bitmap from offset dq - 63 upward: bit x <-> key 63 - x
      const int base = i0w - j0 - (kBN - 1);
      const bool up = ((base & 31) + ql) >= 32;  // this lane's window starts one word on
      const uint32_t b0 = up ? w.o[1] : w.o[0], b1 = up ? w.o[2] : w.o[1], b2 = up ? w.o[3] : w.o[2];
      const int sh = (dq - (kBN - 1)) & 31;
      const uint32_t l0 = __builtin_amdgcn_alignbit(b1, b0, sh);
      const uint32_t l1 = __builtin_amdgcn_alignbit(b2, b1, sh);
      uint32_t k0 = __builtin_bitreverse32(l1);
      uint32_t k1 = __builtin_bitreverse32(l0);
      // columns are visible up to key dq
      const uint32_t c0 = dq >= 31 ? ~0u : (dq < 0 ? 0u : ((2u << dq) - 1u));
      const uint32_t c1 = dq >= 63 ? ~0u : (dq < 32 ? 0u : ((2u << (dq - 32)) - 1u));
      k0 |= w.v[0] & c0;
      k1 |= w.v[1] & c1;
      kh0 = __builtin_amdgcn_alignbit(k1, k0, 4 * half);
      kh1 = k1 >> (4 * half);
    };
    // gathered chunk: its 64 keys ascend (padding n sorts last), so the visible
    // ones are a prefix; a chunk that ends at or before the wave's first row is
    // visible whole, which skips the search for all but the chunks at the
    // diagonal
    auto key_word_chunk = [&](const int* keys, uint32_t& kh0, uint32_t& kh1) {
      int cnt = kBN;
      if (keys[kBN - 1] > i0w) {
        int lo = 0;
#pragma unroll
        for (int step = 32; step > 0; step >>= 1)
          if (keys[lo + step - 1] <= qrow) lo += step;
        cnt = lo + (lo == 63 && keys[63] <= qrow ? 1 : 0);
      }
      const uint32_t k0 = cnt >= 32 ? ~0u : ((1u << cnt) - 1u);
      const uint32_t k1 = cnt >= 64 ? ~0u : (cnt <= 32 ? 0u : ((1u << (cnt - 32)) - 1u));
      kh0 = __builtin_amdgcn_alignbit(k1, k0, 4 * half);
      kh1 = k1 >> (4 * half);
    };

    // ---- matrix-core operands.  Per-lane LDS byte offsets (within kv_lds) of
    // the reads in stage 0; other stages add a multiple of TILEB as an
    // immediate.
    int koff[KS];  // K rows ql (+32 via the immediate), chunk 2*kk + half
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) koff[kk] = KREG + ql * ROWB + 16 * ((2 * kk + half) ^ swz<D>(ql));
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
          voff[part][dt] = VREG + row * ROWB + 16 * (chunk ^ swz<D>(row)) + 8 * (pp & 1);
        }
    }
    typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    f32x16 c0, c1;  // S^T of the tile whose softmax is next
    uint32_t pk[16];  // its probabilities as bf16 pairs (the P^T operand)
    // M half: O^T += V^T(V stage vs) P^T, then S^T = K(K stage ks) Q^T, as
    // one sequence of matrix products.  Product i's LDS operand goes into
    // ring[i % (kAhead + 1)] kAhead products before it runs, so the reads stay
    // ahead of the matrix cores across the switch from PV to QK.
    constexpr int NPV = 4 * DT, NQK = 2 * KS, kAhead = 5;
    auto mhalf = [&](int vs, int ks) {
      u32x4 ring[kAhead + 1];
      auto fetch = [&](int i) {
        u32x4& dst = ring[i % (kAhead + 1)];
        if (i < NPV) {  // PV product: 16-key chunk c4, head dims 32*dt ..
          const int c4 = i / DT, dt = i % DT;
          const int o = vs * TILEB + c4 * 16 * ROWB;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(kv_base + voff[0][dt] + o));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(kv_base + voff[1][dt] + o));
          dst = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {  // QK product: k-step kk, key half h
          const int j = i - NPV, kk = j >> 1, h = j & 1;
          dst = *(const __attribute__((address_space(3))) u32x4*)(kv_base + koff[kk] + ks * TILEB + h * 32 * ROWB);
        }
      };
#pragma unroll
      for (int e = 0; e < 16; ++e) c0[e] = c1[e] = 0.f;
#pragma unroll
      for (int i = 0; i < kAhead; ++i) fetch(i);
#pragma unroll
      for (int i = 0; i < NPV + NQK; ++i) {
        if (i + kAhead < NPV + NQK) fetch(i + kAhead);
        const bf16x8 a = as_bf16x8(ring[i % (kAhead + 1)]);
        if (i < NPV) {
          const int c4 = i / DT, dt = i % DT;
          const bf16x8 pf = as_bf16x8(u32x4{pk[4 * c4], pk[4 * c4 + 1], pk[4 * c4 + 2], pk[4 * c4 + 3]});
          acc[dt] = mfma32(a, pf, acc[dt]);
        } else {
          const int j = i - NPV, kk = j >> 1;
          if (j & 1) c1 = mfma32(a, qf[kk], c1);
          else c0 = mfma32(a, qf[kk], c0);
        }
      }
      // keep that order through scheduling: the first kAhead operands' reads,
      // then per product the reads kAhead ahead and the product itself
      __builtin_amdgcn_sched_group_barrier(0x080, MhalfOrder<NPV, NQK, kAhead>::prologue_reads(), 0);
      MhalfOrder<NPV, NQK, kAhead>::template emit<0>();
    };
    // S^T(K stage 0) alone, for the first tile of a run
    auto qk0 = [&]() {
#pragma unroll
      for (int e = 0; e < 16; ++e) c0[e] = c1[e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 a0 = *(const lds_bf16x8*)(kv_base + koff[kk]);
        const bf16x8 a1 = *(const lds_bf16x8*)(kv_base + koff[kk] + 32 * ROWB);
        c0 = mfma32(a0, qf[kk], c0);
        c1 = mfma32(a1, qf[kk], c1);
      }
    };
    // online softmax of S = (c0, c1) under the key words, in two parts so
    // that other work of the vector half can sit between them.  probs() forms
    // the probabilities against the running maximum as bf16 pairs in pk (the
    // P^T operand), masks them by mode:
    //   kMasked  every tile is masked;
    //   kTested  a tile whose key words cover all its keys in every lane (the
    //            element bits 0x0F0F0F0F of both words) skips the masks;
    //   kNoMask  the caller knows every key of the tile is selected for every
    //            row, so the key words are not even formed;
    // and returns the sum of the lane's share of them.
    // commit() makes sure none of them exceeded kPMax -- the lane's sum of
    // non-negative p bounds each, so the tile's own maximum is needed only
    // when a sum exceeds that (always on a row's first tile, where the running
    // maximum is still kNoMax, and rarely afterwards); then it moves the
    // running maximum, rescales O and the row sum, and forms the tile again.
    // Finally it adds the tile's sum to the row's.  Deciding on the sum, after
    // the next tile's key word and loads are issued, keeps both the maxima and
    // the wait for the sums off the critical path.
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    // Masking.  Element e of c0 (c1) is key word bit 8*(e>>2) + (e&3) of kc0
    // (kc1).  mask_s() sets the scores of unselected keys to -inf, for the
    // maximum; the common path masks the packed probabilities instead, two at
    // a time: pair e of pk (elements 2e, 2e+1) sits at bits b, b+1 with
    // b = 8*(e>>1) + 2*(e&1), and pairs e and e+4 are 16 bits apart.  Shifted
    // left by 15-b the word has bit b at 15 and b+16 at 31; by 14-b, bit b+1 at
    // 15 and b+17 at 31.  v_perm's sign-replicating selectors (8, 9: bits 15
    // and 31 of the low source; 10, 11: of the high source) spread each pair's
    // two bits over the two bf16 halves of a mask word: 24 operations for 16
    // elements instead of 32.
    auto needs_mask = [&](uint32_t kc0, uint32_t kc1, auto mode_c) -> bool {
      constexpr int MODE = decltype(mode_c)::value;
      if constexpr (MODE == kTested)
        return __builtin_amdgcn_ballot_w64((kc0 & kc1 & 0x0F0F0F0Fu) != 0x0F0F0F0Fu) != 0;
      return MODE == kMasked;
    };
    auto mask_s = [&](uint32_t kc0, uint32_t kc1) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int bpos = 8 * (e >> 2) + (e & 3);
        const uint32_t m0 = (uint32_t)__builtin_amdgcn_sbfe((int)kc0, bpos, 1);
        const uint32_t m1 = (uint32_t)__builtin_amdgcn_sbfe((int)kc1, bpos, 1);
        c0[e] = __uint_as_float((m0 & __float_as_uint(c0[e])) | (~m0 & 0xff800000u));
        c1[e] = __uint_as_float((m1 & __float_as_uint(c1[e])) | (~m1 & 0xff800000u));
      }
    };
    auto mask_p = [&](uint32_t kc, uint32_t* w) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = 8 * (j >> 1) + 2 * (j & 1);
        const uint32_t lo = kc << (15 - b), hi = kc << (14 - b);
        w[j] &= __builtin_amdgcn_perm(hi, lo, 0x0A0A0808u);
        w[j + 4] &= __builtin_amdgcn_perm(hi, lo, 0x0B0B0909u);
      }
    };
    // the probabilities of S, masked by the key words where `masked`
    auto form_probs = [&](bool masked, uint32_t kc0, uint32_t kc1) -> float {
      const float nm = -m_run;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pk[e] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(c0[2 * e], cpos, nm)),
                          __builtin_amdgcn_exp2f(fmaf(c0[2 * e + 1], cpos, nm)));
        pk[8 + e] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(c1[2 * e], cpos, nm)),
                              __builtin_amdgcn_exp2f(fmaf(c1[2 * e + 1], cpos, nm)));
      }
      if (masked) {
        mask_p(kc0, pk);
        mask_p(kc1, pk + 8);
      }
      float ts[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 16; ++e)
        ts[e & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e]), ones, ts[e & 3], false);
      return (ts[0] + ts[1]) + (ts[2] + ts[3]);
    };
    auto probs = [&](uint32_t kc0, uint32_t kc1, auto mode_c) -> float {
      return form_probs(needs_mask(kc0, kc1, mode_c), kc0, kc1);
    };
    auto commit = [&](float t, uint32_t kc0, uint32_t kc1, auto mode_c) {
      if (__builtin_amdgcn_ballot_w64(!(t <= kPMax))) {
        if (needs_mask(kc0, kc1, mode_c)) mask_s(kc0, kc1);
        float mx = c0[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = __builtin_elementwise_maximum(mx, c0[e]);
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = __builtin_elementwise_maximum(mx, c1[e]);
        mx = half_max(mx);
        const float mnew = fmaxf(m_run, mx * cpos);
        const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[dt][e] *= alpha;
        m_run = mnew;
        t = form_probs(false, 0u, 0u);  // S is masked already
      }
      l_run += t;
    };

    auto hold_dma_offsets = [&]() {
      if constexpr (!F32) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) asm volatile("" ::"v"(dma_off[0][i]), "v"(dma_off[1][i]));
      }
    };
    constexpr int kDmaPerStep = 2 * NDMA;  // K and V loads one step issues
    const bool lead = wave < kWaves / 2;   // waves w and w + 4 share a SIMD

    // ---- ping-pong pipeline over T tiles.  Tile t's K sits in K stage t % NST
    // and its V in V stage t % NST.  Work on a tile splits into
    //   V(t): the softmax of S(t) into P(t), the key word of tile t+1, and the
    //         loads of K(t+3) and V(t+2);
    //   M(t): O += V(t) P(t) and S(t+1) = K(t+1) Q^T on the matrix cores.
    // Waves 0-3 run V(t) then M(t); waves 4-7 run half a step behind, so each
    // SIMD overlaps one wave's vector work with the other's matrix work.  Every
    // half ends at a workgroup barrier, and after each M half a wave waits
    // until at most its newest step of loads is in flight.  With the half-step
    // offset this completes K(t+1) and V(t) at the barrier before either group
    // first reads them, and no stage is refilled before both groups have
    // finished reading it.
    //
    // `src` supplies the tiles: stage_first() loads K(0..2) and V(0..1),
    // key_word_first() gives the key word of tile 0; within V(t), begin()
    // starts the fetches step t needs, key_word() gives the key word of tile
    // t+1, stage_k()/stage_v() load K(t+3) / V(t+2), and rotate() moves on.
    // Tiles past the end read as zeros and have empty key words.  `mode_c`
    // picks the softmax masking (kNoMask skips the key words altogether).
    auto pipeline = [&](auto& src, int T, auto mode_c) {
      constexpr int MODE = decltype(mode_c)::value;
      load_q();
      src.stage_first();
      uint32_t kc0 = ~0u, kc1 = ~0u;
      if constexpr (MODE != kNoMask) src.key_word_first(kc0, kc1);
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      __syncthreads();
      qk0();
      if (!lead) __syncthreads();  // the half-step offset
      int t = 0;
      auto step = [&](auto s_const) -> bool {
        constexpr int S = decltype(s_const)::value;
        // V(t), at raised issue priority: the vector half is the longer chain,
        // so the SIMD's other wave (in its matrix half) takes the slots it leaves
        __builtin_amdgcn_s_setprio(3);
        src.begin();
        // Block-mode tiles are scattered key blocks whose loads more often
        // reach HBM: issued first thing they gain the softmax's time (3.8 %
        // on the 128K block layer); the vertical-slash tiles, mostly served
        // by L2, are 0.4 % faster issued after it.
        if constexpr (BLK) {
          src.stage_k(KREG + ((S + 3) % NST) * TILEB);
          src.stage_v(VREG + ((S + 2) % NST) * TILEB);
        }
        const float tsum = probs(kc0, kc1, mode_c);
        const uint32_t tk0 = kc0, tk1 = kc1;  // tile t's key words, for commit()
        if constexpr (MODE != kNoMask) src.key_word(kc0, kc1);
        if constexpr (!BLK) {
          src.stage_k(KREG + ((S + 3) % NST) * TILEB);
          src.stage_v(VREG + ((S + 2) % NST) * TILEB);
        }
        commit(tsum, tk0, tk1, mode_c);
        hold_dma_offsets();
        src.rotate();
        // P(t) is finished here, in the vector half, not under the products
#pragma unroll
        for (int e = 0; e < 16; ++e) asm volatile("" : "+v"(pk[e]));
        __syncthreads();
        // M(t)
        __builtin_amdgcn_s_setprio(0);
        mhalf(S, (S + 1) % NST);
        // and S(t+1) is complete before the next vector half starts
        asm volatile("" : "+v"(c0), "+v"(c1));
        if constexpr (F32) __builtin_amdgcn_s_waitcnt(0x0F70);
        else __builtin_amdgcn_s_waitcnt(0x0F70 | kDmaPerStep);
        __syncthreads();
        return ++t < T;
      };
      while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{}) &&
             step(std::integral_constant<int, 2>{}) && step(std::integral_constant<int, 3>{})) {
      }
      if (lead) __syncthreads();  // matches the trailing group's extra barrier
      // drain: every outstanding load lands before the stages are reused
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      __syncthreads();
    };

    // tiles not known to be full: masked, or tested for fullness first where
    // nearly all of them are full
    const std::integral_constant<int, FULL ? kTested : kMasked> rest_mode{};
    const std::integral_constant<int, kNoMask> full_mode{};

    if constexpr (BLK) {
      // ---- block mode: whole 64-key tiles.  The workgroup's rows fall in
      // query blocks qb0 .. qb1 (at most four); its tile list is the union of
      // their kept key blocks at or below each one's diagonal, in ascending
      // order, each entry carrying in bits 24.. which of the query blocks keep
      // it.  A wave's rows lie in one query block, so a tile is either in its
      // set or not, and inside it only the causal mask applies.
      const int qb0 = i0 / kBN, qb1 = i1 / kBN;
      const int nbk = (n + kBN - 1) / kBN;
      const uint32_t* mrow = p.blk + ((size_t)g * nbk + qb0) * p.blk_wpr;
      const int nwords = qb1 / 32 + 1;
      // kept blocks of word w for the query blocks of this workgroup, and the
      // per-query-block words (masked to blocks at or below that query block)
      auto word_of = [&](int r, int w) -> uint32_t {
        const int I = qb0 + r;
        const int lo = 32 * w;
        const uint32_t causal = I >= lo + 31 ? ~0u : (I < lo ? 0u : ((2u << (I - lo)) - 1u));
        return mrow[(size_t)r * p.blk_wpr + w] & causal;
      };
      auto union_word = [&](int w) -> uint32_t {
        uint32_t u = 0u;
        for (int r = 0; r <= qb1 - qb0; ++r) u |= word_of(r, w);
        return u;
      };
      const int tend = nbk;  // a tile index past the keys, in no query block's set
      const int msh = 24 + (i0w / kBN - qb0);
      auto key_word_block = [&](int code, uint32_t& kh0, uint32_t& kh1) {
        const int dq = qrow - (code & 0xFFFFFF) * kBN;  // largest causal key index of this row
        uint32_t k0 = dq >= 31 ? ~0u : (dq < 0 ? 0u : ((2u << dq) - 1u));
        uint32_t k1 = dq >= 63 ? ~0u : (dq < 32 ? 0u : ((2u << (dq - 32)) - 1u));
        if (!((code >> msh) & 1)) k0 = k1 = 0u;
        kh0 = __builtin_amdgcn_alignbit(k1, k0, 4 * half);
        kh1 = k1 >> (4 * half);
      };
      struct BlockSrc {
        decltype(stage_tile)& stage_fn;
        decltype(key_word_block)& key_fn;
        const int* list;
        int T, tend;
        int t, c1, c2, c3, pref;
        __device__ int code(int i) const {
          const int x = __builtin_amdgcn_readfirstlane(list[min(i, T - 1)]);
          return i < T ? x : tend;
        }
        __device__ void stage_first() {
          const int c0 = code(0);
          c1 = code(1);
          c2 = code(2);
          c3 = code(3);
          t = 0;
          stage_fn(0, c0 & 0xFFFFFF, KREG);
          stage_fn(0, c1 & 0xFFFFFF, KREG + TILEB);
          stage_fn(0, c2 & 0xFFFFFF, KREG + 2 * TILEB);
          stage_fn(1, c0 & 0xFFFFFF, VREG);
          stage_fn(1, c1 & 0xFFFFFF, VREG + TILEB);
        }
        __device__ void key_word_first(uint32_t& k0, uint32_t& k1) { key_fn(code(0), k0, k1); }
        __device__ void begin() { pref = list[min(t + 4, T - 1)]; }
        __device__ void key_word(uint32_t& k0, uint32_t& k1) { key_fn(c1, k0, k1); }
        __device__ void stage_k(int dst) { stage_fn(0, c3 & 0xFFFFFF, dst); }
        __device__ void stage_v(int dst) { stage_fn(1, c2 & 0xFFFFFF, dst); }
        __device__ void rotate() {
          c1 = c2;
          c2 = c3;
          const int x = __builtin_amdgcn_readfirstlane(pref);
          c3 = t + 4 < T ? x : tend;
          ++t;
        }
      };
      // lists in windows of kListCap tiles; the pass that fills a window also
      // counts them all, so a list that fits takes one pass over the mask
      for (int wst = 0;; wst += kListCap) {
        int base = 0;
        for (int w0 = 0; w0 < nwords; w0 += kThreads) {
          const int w = w0 + tid;
          const uint32_t u = w < nwords ? union_word(w) : 0u;
          int tot;
          int pos = base + block_excl_scan<kThreads>(__popc(u), &tot, wcnt) - wst;
          for (uint32_t rest = u; rest && pos < kListCap; rest &= rest - 1u) {
            const int bit = __builtin_ctz(rest);
            if (pos >= 0) {
              int memb = 0;
              for (int r = 0; r <= qb1 - qb0; ++r) memb |= (int)((word_of(r, w) >> bit) & 1u) << r;
              glist[pos] = (32 * w + bit) | (memb << 24);
            }
            ++pos;
          }
          base += tot;
        }
        __syncthreads();
        if (base <= wst) break;
        const int T = min(base - wst, kListCap);
        BlockSrc src{stage_tile, key_word_block, glist, T, tend, 0, 0, 0, 0, 0};
        pipeline(src, T, rest_mode);
        n_dense += T;
        if (wst + kListCap >= base) break;
      }
    } else {
      // ---- contiguous tiles: the key ranges the slash clusters reach, in
      // ascending key order.  Cluster ranges are disjoint (clusters are split
      // wherever neighbouring offsets differ by more than bmp + 63), so the list
      // is their concatenation; it is built in LDS windows of kListCap tiles.
      const int32_t* clo = p.clLo + (size_t)wr * p.cap_s;
      const int32_t* chi = p.clHi + (size_t)wr * p.cap_s;
      int ncb;  // clusters whose smallest offset is at most i1
      {
        const int ncl = ldc(p.counts, 4 * wr + 2);
        int lo = 0, hi = ncl;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (ldc(clo, mid) <= i1) lo = mid + 1;
          else hi = mid;
        }
        ncb = lo;
      }
      const int tend = (n + kBN - 1) / kBN;  // a tile index past the keys
      // the j-th cluster in key order covers tiles [tlo, thi]; in a full block
      // every one of them is active, in the short last block they are tested
      auto cluster_tiles = [&](int j, int& tlo, int& thi) {
        const int c = ncb - 1 - j;
        tlo = max(0, i0 - chi[c]) / kBN;
        thi = (i1 - clo[c]) / kBN;
        if (j > 0) tlo = max(tlo, (i1 - clo[c + 1]) / kBN + 1);
      };
      auto active_count = [&](int tlo, int thi) -> int {
        if (!partial) return max(0, thi - tlo + 1);
        int k = 0;
        for (int t = tlo; t <= thi; ++t) k += tile_active(t) ? 1 : 0;
        return k;
      };
      // When the j-th cluster has no gap (every offset from its smallest lo to
      // its largest hi is selected), its tiles [f0, f1] hold only selected
      // pairs for every row of the block: tile T needs the offsets
      // i0 - 64T - 63 .. i1 - 64T, which lie in [lo, hi] exactly for those T
      // (and are then all non-negative, so the tile is causal too).  They run
      // first, unmasked; otherwise f0 = thi + 1, f1 = thi.
      auto floor_div = [](int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); };
      auto cluster_full = [&](int j, int tlo, int thi, int& f0, int& f1) {
        const int c = ncb - 1 - j;
        const int lo = clo[c], hi = chi[c];
        f0 = thi + 1;
        f1 = thi;
        if (prefix(hi + 1) - prefix(lo) != hi - lo + 1) return;
        const int a = max(tlo, floor_div(i1 - hi + kBN - 1, kBN));
        const int b = min(thi, floor_div(i0 - (kBN - 1) - lo, kBN));
        if (a <= b) {
          f0 = a;
          f1 = b;
        }
      };
      int T_total = 0, T_full = 0;
      for (int j0 = 0; j0 < ncb; j0 += kThreads) {
        int cnt = 0, cntf = 0;
        if (j0 + tid < ncb) {
          int tlo, thi, f0, f1;
          cluster_tiles(j0 + tid, tlo, thi);
          cluster_full(j0 + tid, tlo, thi, f0, f1);
          cntf = f1 - f0 + 1;
          cnt = active_count(tlo, thi) - cntf;
        }
        int tot, totf;
        block_excl_scan<kThreads>(cnt, &tot, wcnt);
        block_excl_scan<kThreads>(cntf, &totf, wcnt);
        T_total += tot;
        T_full += totf;
      }
      // Tile codes for steps t+1, t+2, t+3 are carried from step to step; the
      // code of t+4 is read from the LDS list one step ahead (unconditionally:
      // past the end it reads a spare entry and is replaced by tend) and the
      // bitmap words of tile t+1 are requested first thing in the V half, so
      // neither wait sits on the critical path.
      struct TileSrc {
        decltype(stage_tile)& stage_fn;
        decltype(load_words)& load_fn;
        decltype(key_word_tile)& key_fn;
        const int* list;
        int T, tend;
        int t, c1, c2, c3, pref;
        BitWords w;
        __device__ int code(int i) const {
          const int x = __builtin_amdgcn_readfirstlane(list[min(i, T - 1)]);
          return i < T ? x : tend;
        }
        __device__ void stage_first() {
          const int c0 = code(0);
          c1 = code(1);
          c2 = code(2);
          c3 = code(3);
          t = 0;
          stage_fn(0, c0, KREG);
          stage_fn(0, c1, KREG + TILEB);
          stage_fn(0, c2, KREG + 2 * TILEB);
          stage_fn(1, c0, VREG);
          stage_fn(1, c1, VREG + TILEB);
          load_fn(c0, w);
        }
        __device__ void key_word_first(uint32_t& k0, uint32_t& k1) { key_fn(code(0), w, k0, k1); }
        __device__ void begin() {
          load_fn(c1, w);
          pref = list[t + 4];
          __builtin_amdgcn_sched_barrier(0);  // both requests go out first
        }
        __device__ void key_word(uint32_t& k0, uint32_t& k1) { key_fn(c1, w, k0, k1); }
        __device__ void stage_k(int dst) { stage_fn(0, c3, dst); }
        __device__ void stage_v(int dst) { stage_fn(1, c2, dst); }
        __device__ void rotate() {
          c1 = c2;
          c2 = c3;
          const int x = __builtin_amdgcn_readfirstlane(pref);
          c3 = t + 4 < T ? x : tend;
          ++t;
        }
      };
      // Writes window [wst, wst + kListCap) of one pass's tile list into glist:
      // the clusters' full ranges [f0, f1] (full = true), or the rest of their
      // tiles.  In a full block a cluster's tiles form one or two ranges, so
      // after a scan of the counts every slot finds its cluster by a binary
      // search over the clusters' first slots and all slots are written in
      // parallel; in the short last block (one per head) each thread lists its
      // clusters' tiles itself, testing each for an active offset.
      auto list_window = [&](bool full, int wst) {
        int base = 0;
        for (int j0 = 0; j0 < ncb; j0 += kThreads) {
          const int nb = min(kThreads, ncb - j0);
          int cnt = 0, tlo = 0, thi = -1, f0 = 0, f1 = -1;
          if (tid < nb) {
            cluster_tiles(j0 + tid, tlo, thi);
            cluster_full(j0 + tid, tlo, thi, f0, f1);
            cnt = full ? f1 - f0 + 1 : active_count(tlo, thi) - (f1 - f0 + 1);
          }
          int tot;
          int pos = base + block_excl_scan<kThreads>(cnt, &tot, wcnt) - wst;
          if (partial) {
            const int a = full ? f0 : tlo, b = full ? f1 : thi;
            for (int t = a; t <= b && pos < kListCap; ++t) {
              if (!full && t == f0) t = f1 + 1;
              if (t > b) break;
              if (!full && !tile_active(t)) continue;
              if (pos >= 0) glist[pos] = t;
              ++pos;
            }
          } else {
            if (tid < nb) {
              cl_pos[tid] = pos;
              cl_a[tid] = full ? f0 : tlo;
              cl_b[tid] = full ? cnt : f0 - tlo;
              cl_c[tid] = f1 + 1;
            }
            __syncthreads();
            const int s1 = min(kListCap, base + tot - wst);
            for (int sl = max(0, base - wst) + tid; sl < s1; sl += kThreads) {
              int lo = 0, hi = nb - 1;  // the last cluster whose first slot is at or before sl
              while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (cl_pos[mid] <= sl) lo = mid;
                else hi = mid - 1;
              }
              const int r = sl - cl_pos[lo];
              glist[sl] = r < cl_b[lo] ? cl_a[lo] + r : cl_c[lo] + (r - cl_b[lo]);
            }
            __syncthreads();
          }
          base += tot;
        }
        __syncthreads();
      };
      // the full tiles, unmasked
      for (int wst = 0; wst < T_full; wst += kListCap) {
        list_window(true, wst);
        const int T = min(T_full - wst, kListCap);
        TileSrc src{stage_tile, load_words, key_word_tile, glist, T, tend, 0, 0, 0, 0, 0, {}};
        pipeline(src, T, full_mode);
        n_dense += T;
      }
      // the rest, masked
      for (int wst = 0; wst < T_total; wst += kListCap) {
        list_window(false, wst);
        const int T = min(T_total - wst, kListCap);
        TileSrc src{stage_tile, load_words, key_word_tile, glist, T, tend, 0, 0, 0, 0, 0, {}};
        pipeline(src, T, rest_mode);
        n_dense += T;
      }

      // ---- gathered tiles: selected columns in no active tile, 64 per tile
      const int32_t* cv = p.cleanV + (size_t)wr * p.cap_v;
      int total_v;
      {
        const int nv = ldc(p.counts, 4 * wr + 1);
        int lo = 0, hi = nv;  // columns <= i1
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (ldc(cv, mid) <= i1) lo = mid + 1;
          else hi = mid;
        }
        total_v = lo;
      }
      auto stage_chunk = [&](const int* list, int which, int t, int nch, int dst) {
        int key[NDMA];
    #pragma unroll
        for (int i = 0; i < NDMA; ++i) key[i] = t < nch ? list[t * kBN + dma_row[i]] : n;
        stage_keys(which, key, dst);
      };
      struct ChunkSrc {
        decltype(stage_chunk)& stage_fn;
        decltype(key_word_chunk)& key_fn;
        const int* list;
        int T, t;
        __device__ void kw(int i, uint32_t& k0, uint32_t& k1) {
          if (i < T) {
            key_fn(list + i * kBN, k0, k1);
          } else {
            k0 = 0u;
            k1 = 0u;
          }
        }
        __device__ void stage_first() {
          t = 0;
          stage_fn(list, 0, 0, T, KREG);
          stage_fn(list, 0, 1, T, KREG + TILEB);
          stage_fn(list, 0, 2, T, KREG + 2 * TILEB);
          stage_fn(list, 1, 0, T, VREG);
          stage_fn(list, 1, 1, T, VREG + TILEB);
        }
        __device__ void key_word_first(uint32_t& k0, uint32_t& k1) { kw(0, k0, k1); }
        __device__ void begin() {}
        __device__ void key_word(uint32_t& k0, uint32_t& k1) { kw(t + 1, k0, k1); }
        __device__ void stage_k(int dst) { stage_fn(list, 0, t + 3, T, dst); }
        __device__ void stage_v(int dst) { stage_fn(list, 1, t + 2, T, dst); }
        __device__ void rotate() { ++t; }
      };
      int cursor = 0;
      while (cursor < total_v) {
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
          const int below_l = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
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
        if (fill == 0) continue;
        // pad the last chunk with n: sorts after every key, reads as zeros
        for (int r = fill + tid; r < ((fill + kBN - 1) / kBN) * kBN; r += kThreads) glist[r] = n;
        __syncthreads();
        const int nch = (fill + kBN - 1) / kBN;
        // chunks whose last column is at or before the block's first row are
        // visible whole to every row; the columns ascend, so they come first
        int nfull = 0;
        for (int step = 32; step > 0; step >>= 1)
          if (nfull + step <= nch && glist[(nfull + step) * kBN - 1] <= i0) nfull += step;
        if (nfull > 0) {
          ChunkSrc src{stage_chunk, key_word_chunk, glist, nfull, 0};
          pipeline(src, nfull, full_mode);
        }
        if (nch > nfull) {
          ChunkSrc src{stage_chunk, key_word_chunk, glist + nfull * kBN, nch - nfull, 0};
          pipeline(src, nch - nfull, rest_mode);
        }
        n_gath += nch;
      }

    }

    // ---------------- finish: normalise, write O and lse
    const float lt = half_sum(l_run);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if constexpr (F32) {
      if (wave_rows && qrow < n) {
        const size_t ro = ((size_t)head * hstride + row0 + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int d0 = 32 * dt + 8 * a + 4 * half;
            *reinterpret_cast<float4*>(static_cast<float*>(p.out) + ro + d0) =
                float4{acc[dt][4 * a] * inv, acc[dt][4 * a + 1] * inv, acc[dt][4 * a + 2] * inv,
                       acc[dt][4 * a + 3] * inv};
          }
      }
    } else {
      // O leaves through LDS (the K/V rings are idle after the last drain
      // barrier): a wave's 32 rows are contiguous in HBM, so after a transpose
      // each store moves whole rows, 1 KiB per instruction, instead of 8-byte
      // pieces of 32 rows.  16-byte chunks are XOR-swizzled by row.
      constexpr int OCH = D / 8;
      lds_u8* const ob = kv_base + wave * 32 * ROWB;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int pc = (4 * dt + a) ^ (ql & (OCH - 1));
          *(__attribute__((address_space(3))) u32x2*)(ob + ql * ROWB + pc * 16 + 8 * half) =
              u32x2{pack_bf16(acc[dt][4 * a] * inv, acc[dt][4 * a + 1] * inv),
                    pack_bf16(acc[dt][4 * a + 2] * inv, acc[dt][4 * a + 3] * inv)};
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's rows are in LDS
      __builtin_amdgcn_wave_barrier();
      constexpr int RPI = 1024 / ROWB;     // rows per store instruction
#pragma unroll
      for (int it = 0; it < 32 / RPI; ++it) {
        const int r = it * RPI + lane / OCH, c = lane % OCH;
        const u32x4 val = *(const __attribute__((address_space(3))) u32x4*)(ob + r * ROWB + 16 * (c ^ (r & (OCH - 1))));
        if (wave_rows && i0w + r < n)
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) +
                                    ((size_t)head * hstride + row0 + i0w + r) * D + 8 * c) = val;
      }
    }
    if (wave_rows && qrow < n && half == 0 && p.lse)
      p.lse[(size_t)head * hstride + row0 + qrow] = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -__builtin_inff();
    if (tid == 0 && p.stats) {
      atomicAdd(&p.stats[0], (unsigned long long)n_dense);
      atomicAdd(&p.stats[1], (unsigned long long)n_gath);
    }
    // the next item; LDS (the rings, the list) is reused only after every
    // wave is past this item's last read of it
    if (tid == 0) {
      long long nx = class_item(cls, claim);
      for (int j = 1; nx >= p.nitems && j < kQueues; ++j) {
        const int c = (cls + j) % kQueues;
        nx = class_item(c, atomicAdd(&p.queue[c], 1u));
      }
      next_item = (int)min(nx, (long long)p.nitems);
    }
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(next_item);
  }
}

int heads_per_block(int group) { return group < kWaves ? group : kWaves; }

// Workgroups of a persistent launch of `kern`: as many as the device holds
// at once (per device, computed once), at most `items`.
template <void (*KERN)(AttnParams)>
unsigned persistent_grid(long long items) {
  static std::atomic<int> slots[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int s = slots[dev].load(std::memory_order_relaxed);
  if (s <= 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, KERN, kThreads, 0) != hipSuccess) occ = 0;
    s = cus > 0 && occ > 0 ? cus * occ : 1024;
    slots[dev].store(s, std::memory_order_relaxed);
  }
  return (unsigned)std::min<long long>(items, s);
}

template <int D, bool F32, bool BLK, bool FULL>
void launch_attn_kernel(const AttnParams& prm, hipStream_t stream) {
  constexpr auto kern = attn_kernel<D, F32, BLK, FULL>;
  hipLaunchKernelGGL(kern, dim3(persistent_grid<kern>(prm.nitems)), dim3(kThreads), 0, stream, prm);
}

// the signed softmax multiplier of a finite scale (see AttnParams::c)
void set_scale(AttnParams& prm, float scale) {
  prm.c = scale == 0.f ? FLT_MIN : scale * kLog2e;
}

}  // namespace

int attn_query_rows_per_block(int group) {
  (void)group;
  return 32 * kWaves;
}

long long attn_workgroups(int group, int sets, long long n) {
  const int hpw = heads_per_block(group);
  const int bmp = 32 * (kWaves / hpw);
  return (n + bmp - 1) / bmp * sets * (group / hpw);
}

namespace {

// A packed batch as one launch: the device sequence table and, per sequence
// in the caller's order, its length (both inside the workspace).
struct Packed {
  const int* tab = nullptr;   // AttnParams::seq_tab (null: one sequence)
  const int* lens = nullptr;  // [nseq] lengths, caller order
  int nrun = 0;               // non-empty sequences, in the table's order
  int sets = 1;               // index-set rows per sequence
  long long wgs = 0;          // workgroups of the attention launch
};

// tile build over `rows` index-set rows (positions below n, or below their
// sequence's length) and the attention launch
hipError_t run_attn(const void* q, const void* k, const void* v, bool f32, int h_q, int h_kv,
                    int rows, int n, int d, float scale, const int32_t* v_idx,
                    const int32_t* v_cnt, int cap_v, const int32_t* s_off, const int32_t* s_cnt,
                    int cap_s, void* out, float* lse, const AttnWsLayout& L, char* base,
                    hipStream_t stream, const AttnLayout& lay, const Packed& pk) {
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

  if (pk.tab) {
    hipLaunchKernelGGL(ws_clear_rows_kernel, dim3((unsigned)rows), dim3(256), 0, stream, bitO,
                       bitV, L.stride, pk.lens, pk.sets, stats);
  } else {
    const size_t nwords = (size_t)rows * L.stride;
    hipLaunchKernelGGL(ws_clear_kernel, dim3((unsigned)std::min<size_t>((nwords + 255) / 256, 2048)),
                       dim3(256), 0, stream, bitO, bitV, nwords, stats);
  }
  const int capm = std::max(cap_v, cap_s);
  hipLaunchKernelGGL(ws_setbits_kernel, dim3((unsigned)rows, (unsigned)std::min((capm + 255) / 256, 4096)),
                     dim3(256), 0, stream, v_idx, v_cnt, cap_v, s_off, s_cnt, cap_s, n, pk.lens,
                     pk.sets, bitO, bitV, L.stride);
  hipLaunchKernelGGL(ws_scan_kernel, dim3((unsigned)rows), dim3(1024), 0, stream, bitO, bitV,
                     L.stride, L.words, prefO, cleanO, cap_s, cleanV, cap_v, counts, pk.lens,
                     pk.sets);
  // offsets closer than bmp + 64 reach one contiguous run of 64-key tiles
  hipLaunchKernelGGL(ws_cluster_kernel, dim3((unsigned)rows), dim3(1024), 0, stream, cleanO,
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
  prm.blk = nullptr;
  prm.blk_wpr = 0;
  prm.kvdiv = lay.kvdiv;
  prm.hstride = lay.hstride ? lay.hstride : n;
  set_scale(prm, scale);
  prm.row0 = lay.row0;
  prm.seq_tab = pk.tab;
  prm.nseq = pk.nrun;
  const long long wgs = pk.tab ? pk.wgs : (long long)prm.nblocks * h_kv * nsplit;
  if (wgs <= 0) return hipSuccess;
  prm.nitems = (int)wgs;
  prm.queue = reinterpret_cast<unsigned*>(stats + 4);
  // a caller that knows most tiles are full (every offset selected) takes
  // the instantiation that skips their masks
  const bool dense = lay.full_tiles;
  if (d == 128) {
    if (dense) {
      if (f32) launch_attn_kernel<128, true, false, true>(prm, stream);
      else launch_attn_kernel<128, false, false, true>(prm, stream);
    } else {
      if (f32) launch_attn_kernel<128, true, false, false>(prm, stream);
      else launch_attn_kernel<128, false, false, false>(prm, stream);
    }
  } else {
    if (dense) {
      if (f32) launch_attn_kernel<64, true, false, true>(prm, stream);
      else launch_attn_kernel<64, false, false, true>(prm, stream);
    } else {
      if (f32) launch_attn_kernel<64, true, false, false>(prm, stream);
      else launch_attn_kernel<64, false, false, false>(prm, stream);
    }
  }
  return hipGetLastError();
}

// copies up to kTabChunk ints from the kernel's arguments into device memory,
// so the sequence table needs no host buffer that outlives the call
constexpr int kTabChunk = 240;
struct TabChunk {
  int v[kTabChunk];
};
__global__ void ws_table_kernel(int* dst, int cnt, TabChunk c) {
  if ((int)threadIdx.x < cnt) dst[threadIdx.x] = c.v[threadIdx.x];
}

}  // namespace

hipError_t launch_attn(const void* q, const void* k, const void* v, bool f32, int h_q, int h_kv,
                       int n, int d, float scale, const int32_t* v_idx, const int32_t* v_cnt,
                       int cap_v, const int32_t* s_off, const int32_t* s_cnt, int cap_s, void* out,
                       float* lse, void* ws, hipStream_t stream, const AttnLayout& lay) {
  const AttnWsLayout L(h_kv, n, cap_v, cap_s);
  return run_attn(q, k, v, f32, h_q, h_kv, h_kv, n, d, scale, v_idx, v_cnt, cap_v, s_off, s_cnt,
                  cap_s, out, lse, L, static_cast<char*>(ws), stream, lay, Packed());
}

int attn_varlen_table_ints(int nseq) { return 5 * (nseq + 1); }

hipError_t launch_attn_varlen(const void* q, const void* k, const void* v, bool f32, int h_q,
                              int sets, int kvdiv, int total_n, int d, float scale,
                              const int32_t* cu_seqlens, int nseq, int max_len,
                              const int32_t* v_idx, const int32_t* v_cnt, int cap_v,
                              const int32_t* s_off, const int32_t* s_cnt, int cap_s, void* out,
                              float* lse, void* ws, hipStream_t stream) {
  const AttnWsLayout L(nseq * sets, max_len, cap_v, cap_s, attn_varlen_table_ints(nseq));
  char* base = static_cast<char*>(ws);
  const int group = h_q / sets;
  const int hpw = heads_per_block(group);
  const int nsplit = group / hpw;
  const int bmp = 32 * (kWaves / hpw);
  // the table: non-empty sequences longest first (their last query blocks
  // carry the most keys), as workgroup starts, lengths, first rows and
  // indices, each nrun + 1 ints; then every sequence's length
  std::vector<int> order;
  for (int s = 0; s < nseq; ++s)
    if (cu_seqlens[s + 1] > cu_seqlens[s]) order.push_back(s);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
    return cu_seqlens[x + 1] - cu_seqlens[x] > cu_seqlens[y + 1] - cu_seqlens[y];
  });
  const int nrun = (int)order.size();
  std::vector<int> tab(4 * (nrun + 1) + nseq, 0);
  long long wg = 0;
  for (int i = 0; i < nrun; ++i) {
    const int s = order[i], len = cu_seqlens[s + 1] - cu_seqlens[s];
    tab[i] = (int)wg;
    tab[(nrun + 1) + i] = len;
    tab[2 * (nrun + 1) + i] = cu_seqlens[s];
    tab[3 * (nrun + 1) + i] = s;
    wg += (long long)((len + bmp - 1) / bmp) * sets * nsplit;
  }
  if (wg >= (1LL << 31)) return hipErrorInvalidValue;
  tab[nrun] = (int)wg;
  for (int s = 0; s < nseq; ++s) tab[4 * (nrun + 1) + s] = cu_seqlens[s + 1] - cu_seqlens[s];
  int* dtab = reinterpret_cast<int*>(base + L.off_tab);
  for (size_t at = 0; at < tab.size(); at += kTabChunk) {
    TabChunk c;
    const int cnt = (int)std::min<size_t>(kTabChunk, tab.size() - at);
    std::copy(tab.begin() + at, tab.begin() + at + cnt, c.v);
    hipLaunchKernelGGL(ws_table_kernel, dim3(1), dim3(256), 0, stream, dtab + at, cnt, c);
  }
  Packed pk;
  pk.tab = dtab;
  pk.lens = dtab + 4 * (nrun + 1);
  pk.nrun = nrun;
  pk.sets = sets;
  pk.wgs = wg;
  AttnLayout lay;
  lay.kvdiv = kvdiv;
  lay.hstride = total_n;
  return run_attn(q, k, v, f32, h_q, sets, nseq * sets, max_len, d, scale, v_idx, v_cnt, cap_v,
                  s_off, s_cnt, cap_s, out, lse, L, base, stream, lay, pk);
}

hipError_t launch_attn_blocks(const void* q, const void* k, const void* v, bool f32, int h_q,
                              int h_kv, int n, int d, float scale, const uint32_t* blk, int wpr,
                              void* out, float* lse, void* ws, hipStream_t stream) {
  unsigned long long* stats = static_cast<unsigned long long*>(ws);
  hipLaunchKernelGGL(ws_clear_kernel, dim3(1), dim3(64), 0, stream, nullptr, nullptr, (size_t)0, stats);
  const int group = h_q / h_kv;
  const int hpw = heads_per_block(group);
  const int nsplit = group / hpw;
  const int bmp = 32 * (kWaves / hpw);
  AttnParams prm = {};
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
  prm.stats = stats;
  prm.blk = blk;
  prm.blk_wpr = wpr;
  prm.kvdiv = 1;
  prm.hstride = n;
  set_scale(prm, scale);
  prm.row0 = 0;
  const long long wgs = (long long)prm.nblocks * h_kv * nsplit;
  if (wgs <= 0) return hipSuccess;
  prm.nitems = (int)wgs;
  prm.queue = reinterpret_cast<unsigned*>(stats + 4);
  if (d == 128) {
    if (f32) launch_attn_kernel<128, true, true, true>(prm, stream);
    else launch_attn_kernel<128, false, true, true>(prm, stream);
  } else {
    if (f32) launch_attn_kernel<64, true, true, true>(prm, stream);
    else launch_attn_kernel<64, false, true, true>(prm, stream);
  }
  return hipGetLastError();
}

}  // namespace vs
