// vs_select.hip -- cumulative-mass budget selection without a sort, gfx950.
//
// VSPrefill (gist.science summaries of arXiv 2603.04460, English page,
// Technical Summary section 2, "3. Adaptive Inference Pipeline, Dynamic
// Budgeting") chooses per layer the fewest top-scored indices whose
// predicted mass reaches a threshold; FlashPrefill's summary (arXiv
// 2603.06199, Spanish page, section 1) notes that sorting and cumulative
// sums are what makes such selection slow on GPUs.  Here the budget is found
// by a most-significant-digit radix select over the order-preserving bits of
// the fp32 score, with one histogram of counts and one of integer masses per
// digit (11, 11 and 10 bits), so no element is ever sorted:
//   1. m = max score; u_c = quantised mass of score_c - m (exact integer);
//      U = sum u; T = ceil(mass * U).  Only scores within 32 of the maximum
//      are candidates (everything else has u = 0 and sorts after the element
//      that completes T).
//   2. Digit by digit from the top of the 32-bit key, the bucket holding the
//      K-th candidate in (score descending, index ascending) order is the
//      first whose running mass reaches T or whose running count reaches cap.
//   3. Equal scores have equal u, so the number r of tied candidates needed
//      is a division; they are the r lowest indices of the tie.
//   4. An ordered compaction writes the chosen candidates ascending.
// Every pass over the candidates is spread over workgroups of kSelChunk
// candidates (a few hundred workgroups at n = 128K) and joined by integer
// atomics in the workspace; integer sums are order-free, so the result does
// not depend on scheduling.  A pass's bucket decision is a scan of its 2048
// bins, cheap enough that every workgroup of the next pass makes it for
// itself instead of waiting for a launch of its own; keys and masses are
// recomputed from the scores in each pass instead of being stored.  The chain
// is five launches: maximum, masses with the first digit, two more digits,
// and the ordered write, in which each chunk publishes its own counts and
// adds those of the chunks before it (counting a chunk itself if its count
// is late, so the result never waits on scheduling).
// The same chain serves FlashPrefill's max-based dynamic threshold
// (FlashPrefill summary, Spanish page, section 2.B): keep the candidates whose
// softmax score is at least alpha times the largest, i.e. u >= ceil(alpha *
// 2^32) (the maximum has u = 2^32), at most cap of them in the same order;
// there the budget is that count and no mass target applies.
// The mass arithmetic follows a fixed specification so the budget is an
// exact integer decision: exp is Cody and Waite's range reduction with a
// two-piece ln 2 (W. J. Cody, W. Waite, 1980) and the degree-7 Taylor
// polynomial by explicit fused multiply-adds in fp32; nothing else is fused.
#include "vs_common.h"
#include "vs_internal.h"

#pragma clang fp contract(off)

namespace vs {

namespace {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kPasses = 3;        // digits of the 32-bit key: bits 21..31, 10..20, 0..9
constexpr int kBins = kSelBins;   // histogram bins of a pass (the last uses 1024)
static_assert(kPasses == kSelDigitPasses, "workspace passes");
constexpr int kBinsPerLane = kBins / 64;

__device__ __forceinline__ int digit_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__device__ __forceinline__ int digit_bits(int p) { return p == 2 ? 10 : 11; }

// per-row state (unsigned 64-bit words in the workspace, kSelStateWords of them)
enum : int {
  kStU = 0,       // sum of quantised masses
  kStAbove,       // candidates at or above the threshold (threshold mode)
  kStDec,         // the decision after digit pass p: 5 words at kStDec + 5 p
  kStEnd = kStDec + 5 * kPasses
};
static_assert(kStEnd <= kSelStateWords, "state words");

__device__ __forceinline__ float spec_exp(float x) {
  const float log2e = 0x1.715476p+0f;
  const float ln2_hi = 0x1.62e4p-1f;
  const float ln2_lo = 0x1.7f7d1cp-20f;
  const float kf = __builtin_rintf(x * log2e);
  float r = __builtin_fmaf(-kf, ln2_hi, x);
  r = __builtin_fmaf(-kf, ln2_lo, r);
  float q = 0x1.a01a02p-13f;
  q = __builtin_fmaf(q, r, 0x1.6c16c2p-10f);
  q = __builtin_fmaf(q, r, 0x1.111112p-7f);
  q = __builtin_fmaf(q, r, 0x1.555556p-5f);
  q = __builtin_fmaf(q, r, 0x1.555556p-3f);
  q = __builtin_fmaf(q, r, 0.5f);
  q = __builtin_fmaf(q, r, 1.0f);
  q = __builtin_fmaf(q, r, 1.0f);
  return __builtin_ldexpf(q, (int)kf);
}

__device__ __forceinline__ uint64_t spec_mass(float x) {
  if (x < -32.0f) return 0ull;
  const double e = (double)spec_exp(x) * 4294967296.0;
  return (uint64_t)__builtin_rint(e);
}

// larger score -> larger key; -0 and +0 share a key
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t b = __float_as_uint(s == 0.0f ? 0.0f : s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ float load_score(const float* row, int n, int kind, int c) {
  return kind == 0 ? row[c] : row[n - 1 - c];
}

// Inclusive scans over a wave's lanes on the data-parallel-primitive moves
// of gfx9: shifts by 1, 2, 4, 8 within each row of 16 lanes, then row 0's
// last lane added to row 1 (and row 2's to row 3), then lane 31 added to
// rows 2 and 3.  Lanes a move does not reach add 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long x) {
  const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)x), hi = dpp_u32<CTRL, ROWS>((uint32_t)(x >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
template <typename T, int CTRL, int ROWS>
__device__ __forceinline__ T dpp_move(T x) {
  if constexpr (sizeof(T) == 8) return (T)dpp_u64<CTRL, ROWS>((unsigned long long)x);
  else return (T)dpp_u32<CTRL, ROWS>((uint32_t)x);
}
// LANES = 64: the whole wave; LANES = 32: each half on its own
template <int LANES, typename T>
__device__ __forceinline__ T wave_scan(T x) {
  x += dpp_move<T, 0x111, 0xf>(x);  // row_shr:1
  x += dpp_move<T, 0x112, 0xf>(x);  // row_shr:2
  x += dpp_move<T, 0x114, 0xf>(x);  // row_shr:4
  x += dpp_move<T, 0x118, 0xf>(x);  // row_shr:8
  x += dpp_move<T, 0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  if constexpr (LANES == 64) x += dpp_move<T, 0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

template <typename T, typename Op>
__device__ T wave_reduce(T x, Op op) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = op(x, __shfl_xor(x, o, 64));
  return x;
}

// block-wide reduction through `sh` (kSelWaves slots); every thread gets it
template <typename T, typename Op>
__device__ T block_reduce(T x, Op op, T* sh) {
  x = wave_reduce(x, op);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
  __syncthreads();
  T r = sh[0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) r = op(r, sh[w]);
  __syncthreads();
  return r;
}

// exclusive count of `flag` over the block in thread order, plus the total
__device__ int block_count(bool flag, int* total, int* sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t bal = __builtin_amdgcn_ballot_w64(flag);
  const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
  if (lane == 0) sh[wv] = __popcll(bal);
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int c = sh[w];
    before += w < wv ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + below;
}

// Workspace rows r < hk select side[0]'s candidates, rows hk .. 2 hk - 1
// side[1]'s (when two kinds share one chain).
struct SelArgs {
  SelSide side[2];
  int hk;  // heads per side
  int n, chunks;
  double mass;
  unsigned long long thresh;  // threshold mode: keep u >= thresh; 0 for the mass budget
  uint32_t* cmax;             // [rows][chunks] largest key of each chunk
  unsigned long long* state;  // [rows][kSelStateWords]
  uint32_t* hcnt;             // [rows][kPasses][kBins]
  unsigned long long* hmass;  // [rows][kPasses][kBins]
  unsigned long long* slot;   // [rows][chunks]: a chunk's published counts (see sel_write_kernel)
};

// what workspace row r selects from and where it writes
struct RowRef {
  const float* row;  // its candidates' scores
  int kind, cap;
  int32_t* idx;      // its [cap] output
  int32_t* count;    // its count
};
__device__ __forceinline__ RowRef row_ref(const SelArgs& a, int r) {
  const int s = r >= a.hk ? 1 : 0, h = r - s * a.hk;
  const SelSide& sd = a.side[s];
  return RowRef{sd.logit + (size_t)h * a.n, sd.kind, sd.cap, sd.idx + (size_t)h * sd.cap, sd.count + h};
}

// The scores of one chunk, with -0 made +0, kPer per thread: thread t holds
// candidates c0 + kSelThreads j + t.  All the loads are issued before any is used,
// so a pass waits for one memory latency instead of kPer; slots past n hold
// NaN (no comparison with NaN is true, so they are never candidates).
constexpr int kPer = kSelChunk / kSelThreads;
__device__ __forceinline__ void load_chunk(const RowRef& rr, int n, int c0, float (&v)[kPer]) {
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int c = c0 + kSelThreads * j + (int)threadIdx.x;
    v[j] = c < n ? load_score(rr.row, n, rr.kind, c) : __builtin_nanf("");
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) v[j] = v[j] == 0.0f ? 0.0f : v[j];
}

// The decision after a digit pass: the digits of the K-th candidate's key
// fixed so far (in place), the mass and count of the candidates whose keys
// are above its bucket, and the bucket's own count and mass.
struct Dec {
  unsigned long long prefix, mass_above, cnt_above, bcnt, bmass;
};

__device__ __forceinline__ Dec load_dec(const unsigned long long* st, int p) {
  const unsigned long long* d = st + kStDec + 5 * p;
  return Dec{d[0], d[1], d[2], d[3], d[4]};
}

__device__ __forceinline__ void store_dec(const SelArgs& a, int r, int p, const Dec& d) {
  unsigned long long* w = a.state + (size_t)kSelStateWords * r + kStDec + 5 * p;
  w[0] = d.prefix;
  w[1] = d.mass_above;
  w[2] = d.cnt_above;
  w[3] = d.bcnt;
  w[4] = d.bmass;
}

// The global values a decision needs, all loaded together at a kernel's
// start (with the chunk's scores) so that the pass waits for one memory
// latency: the row's U and threshold count, the decision before the one to
// make, this thread's share of the histogram it is made on, and the chunks'
// largest keys.
constexpr int kBinsPerThread = kBins / kSelThreads;
struct Pre {
  unsigned long long U, above;
  Dec prev;
  uint32_t hc[kBinsPerThread];
  unsigned long long hm[kBinsPerThread];
  uint32_t cm;  // the largest of this thread's chunks' largest keys
};

// prefetch for the decision after digit pass pd (pd < 0: none, only the
// chunks' largest keys)
__device__ __forceinline__ void prefetch(const SelArgs& a, int r, int pd, Pre& f) {
  const unsigned long long* st = a.state + (size_t)kSelStateWords * r;
  f.cm = 0u;
  for (int i = threadIdx.x; i < a.chunks; i += kSelThreads) f.cm = max(f.cm, a.cmax[(size_t)r * a.chunks + i]);
  if (pd < 0) return;
  f.U = st[kStU];
  f.above = st[kStAbove];
  f.prev = pd > 0 ? load_dec(st, pd - 1) : Dec{0ull, 0ull, 0ull, 0ull, 0ull};
  const uint32_t* hc = a.hcnt + ((size_t)r * kPasses + pd) * kBins;
  const unsigned long long* hm = a.hmass + ((size_t)r * kPasses + pd) * kBins;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) {
    f.hc[i] = hc[kSelThreads * i + threadIdx.x];
    f.hm[i] = hm[kSelThreads * i + threadIdx.x];
  }
}

// the prefetched histogram into LDS
__device__ __forceinline__ void stage_hist(const Pre& f, uint32_t* lc, unsigned long long* lm) {
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) {
    lc[kSelThreads * i + threadIdx.x] = f.hc[i];
    lm[kSelThreads * i + threadIdx.x] = f.hm[i];
  }
}

// the mass target and the count the selection may take
__device__ __forceinline__ void target_of(const SelArgs& a, unsigned long long U, unsigned long long above,
                                          int r, unsigned long long& T, unsigned long long& cap) {
  if (a.thresh) {
    // threshold mode: the budget is the count at or above the threshold; no
    // mass target can stop the walk first (T exceeds the total mass)
    T = U + 1ull;
    cap = min((unsigned long long)row_ref(a, r).cap, above);
  } else {
    T = (unsigned long long)__builtin_ceil(a.mass * (double)U);
    cap = (unsigned long long)row_ref(a, r).cap;
  }
}

// Pass p's decision, from its complete histogram (staged in LDS by
// stage_hist, and visible to the first wave) and the decision before it,
// made by the block's first wave and handed to every thread through LDS.
// Digits are walked from the top down (descending keys): the bucket taken is
// the first whose running mass reaches T or running count reaches cap.  Two
// scans: over the lanes' sums of 32 bins, then over the 32 bins of the lane
// where the running total is reached.
__device__ Dec decide(const SelArgs& a, int r, int p, const Pre& f, const uint32_t* lc,
                      const unsigned long long* lm, Dec* sh) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    unsigned long long T, cap;
    target_of(a, f.U, f.above, r, T, cap);
    const Dec& prev = f.prev;
    // lane l sums digits top - kBinsPerLane l .. (descending), in an order
    // rotated by the lane so that the lanes' LDS reads fall in distinct banks
    // (all reads issued before the first add, so their latencies overlap)
    const int top = kBins - 1 - kBinsPerLane * lane;
    uint32_t cv[kBinsPerLane];
    unsigned long long mv[kBinsPerLane];
#pragma unroll
    for (int i = 0; i < kBinsPerLane; ++i) {
      const int b = top - ((i + lane) & (kBinsPerLane - 1));
      cv[i] = lc[b];
      mv[i] = lm[b];
    }
    unsigned long long bc = 0, bm = 0;
#pragma unroll
    for (int i = 0; i < kBinsPerLane; ++i) {
      bc += cv[i];
      bm += mv[i];
    }
    const unsigned long long sc = wave_scan<64>(bc), sm = wave_scan<64>(bm);  // inclusive, over lanes
    const bool hit = (prev.mass_above + sm >= T) || (prev.cnt_above + sc >= cap);
    const uint64_t hb = __builtin_amdgcn_ballot_w64(hit);
    const int L = hb ? __builtin_ctzll(hb) : 63;
    // the lane's 32 bins, one per lane, on top of everything before lane L
    auto lane_u64 = [](unsigned long long x, int l) {
      return ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), l) << 32) |
             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
    };
    const unsigned long long base_c = prev.cnt_above + lane_u64(sc - bc, L);
    const unsigned long long base_m = prev.mass_above + lane_u64(sm - bm, L);
    const int dg = kBins - 1 - kBinsPerLane * L - (lane & (kBinsPerLane - 1));
    const unsigned long long oc = lc[dg], om = lm[dg];
    static_assert(kBinsPerLane == 32, "the second scan covers one half-wave");
    const unsigned long long ic = wave_scan<32>(oc), im = wave_scan<32>(om);  // over the 32 bins
    const bool hit2 = lane < kBinsPerLane && (base_m + im >= T || base_c + ic >= cap);
    const uint64_t hb2 = __builtin_amdgcn_ballot_w64(hit2);
    const int j = hb2 ? __builtin_ctzll(hb2) : kBinsPerLane - 1;
    if (lane == j) {
      *sh = Dec{prev.prefix | ((unsigned long long)dg << digit_shift(p)), base_m + im - om,
                base_c + ic - oc, oc, om};
    }
  }
  __syncthreads();
  const Dec d = *sh;
  __syncthreads();
  return d;
}

// 1. largest key of each chunk; the row's chunks also clear its state, its
//    histograms and its published counts for the passes that follow
__global__ __launch_bounds__(kSelThreads) void sel_max_kernel(SelArgs a) {
  __shared__ uint32_t sh[kSelWaves];
  const int r = blockIdx.y, q = blockIdx.x, c0 = q * kSelChunk;
  const RowRef rr = row_ref(a, r);
  float v[kPer];
  load_chunk(rr, a.n, c0, v);
  const int stride = a.chunks * kSelThreads;
  for (int i = q * kSelThreads + threadIdx.x; i < kPasses * kBins; i += stride) {
    a.hcnt[(size_t)r * kPasses * kBins + i] = 0u;
    a.hmass[(size_t)r * kPasses * kBins + i] = 0ull;
  }
  if (q == 0)
    for (int i = threadIdx.x; i < kSelStateWords; i += kSelThreads) a.state[(size_t)kSelStateWords * r + i] = 0ull;
  for (int i = q * kSelThreads + threadIdx.x; i < a.chunks; i += stride) a.slot[(size_t)r * a.chunks + i] = 0ull;
  uint32_t km = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (c0 + kSelThreads * j + (int)threadIdx.x < a.n) km = max(km, order_key(v[j]));
  km = block_reduce(km, [](uint32_t x, uint32_t y) { return max(x, y); }, sh);
  if (threadIdx.x == 0) a.cmax[(size_t)r * a.chunks + q] = km;
}

// the row's maximum score, from the chunks' largest keys
__device__ float row_max(const Pre& f, uint32_t* sh) {
  const uint32_t km = block_reduce(f.cm, [](uint32_t x, uint32_t y) { return max(x, y); }, sh);
  return key_score(km);
}

// 2. digit pass p over one chunk.  Pass 0 also forms every candidate's
//    quantised mass and adds U and the threshold count; later passes first
//    make the previous pass's decision (block 0 of the row stores it) and
//    histogram only the candidates whose higher digits match it.
__global__ __launch_bounds__(kSelThreads) void sel_hist_kernel(SelArgs a, int p) {
  __shared__ uint32_t lc[kBins];
  __shared__ unsigned long long lm[kBins];
  __shared__ unsigned long long shu[kSelWaves];
  __shared__ uint32_t shk[kSelWaves];
  __shared__ Dec shd;
  const int r = blockIdx.y, q = blockIdx.x, c0 = q * kSelChunk;
  const RowRef rr = row_ref(a, r);
  unsigned long long* st = a.state + (size_t)kSelStateWords * r;
  float v[kPer];
  load_chunk(rr, a.n, c0, v);
  Pre f;
  prefetch(a, r, p - 1, f);
  if (p > 0) stage_hist(f, lc, lm);
  const float mx = row_max(f, shk);  // its barrier also completes the staging
  unsigned long long hi = 0ull;  // the digits above this pass's, where they must match
  if (p > 0) {
    const Dec d = decide(a, r, p - 1, f, lc, lm, &shd);
    if (q == 0 && threadIdx.x == 0) store_dec(a, r, p - 1, d);
    hi = d.prefix;
  }
  for (int i = threadIdx.x; i < kBins; i += kSelThreads) {
    lc[i] = 0u;
    lm[i] = 0ull;
  }
  __syncthreads();
  const int shift = digit_shift(p), top = shift + digit_bits(p);
  const uint32_t dmask = (1u << digit_bits(p)) - 1u;
  unsigned long long usum = 0, nabove = 0;
  // Candidates usually crowd into a few digits, and LDS atomics on one
  // address serialise; each lane keeps the digit of its first candidate in
  // registers and sends only the others to LDS as they come.
  int rd = -1;
  uint32_t rc = 0u;
  unsigned long long rm = 0ull;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const float s = v[j];
    const float x = s - mx;
    if (!(x >= -32.0f)) continue;  // not a candidate
    const uint32_t k = order_key(s);
    if (p > 0 && ((unsigned long long)k >> top) != (hi >> top)) continue;
    const uint64_t u = spec_mass(x);
    if (p == 0) {
      usum += u;
      nabove += (a.thresh && u >= a.thresh) ? 1ull : 0ull;
    }
    const int dg = (int)((k >> shift) & dmask);
    if (rd < 0) rd = dg;
    if (dg == rd) {
      rc += 1u;
      rm += u;
    } else {
      atomicAdd(&lc[dg], 1u);
      atomicAdd(&lm[dg], (unsigned long long)u);
    }
  }
  if (rd >= 0) {
    atomicAdd(&lc[rd], rc);
    atomicAdd(&lm[rd], rm);
  }
  if (p == 0) {
    usum = block_reduce(usum, [](unsigned long long x, unsigned long long y) { return x + y; }, shu);
    nabove = block_reduce(nabove, [](unsigned long long x, unsigned long long y) { return x + y; }, shu);
    if (threadIdx.x == 0) {
      atomicAdd(&st[kStU], usum);
      if (a.thresh) atomicAdd(&st[kStAbove], nabove);
    }
  }
  __syncthreads();
  uint32_t* hc = a.hcnt + ((size_t)r * kPasses + p) * kBins;
  unsigned long long* hm = a.hmass + ((size_t)r * kPasses + p) * kBins;
  for (int i = threadIdx.x; i < kBins; i += kSelThreads)
    if (lc[i]) {
      atomicAdd(&hc[i], lc[i]);
      atomicAdd(&hm[i], lm[i]);
    }
}

// a chunk's counts as published: bit 63 set, then the ties with the K-th key
// in bits 32..62 and the candidates above it in bits 0..31
constexpr unsigned long long kSlotValid = 1ull << 63;
constexpr int kSpinLimit = 4096;  // polls of a late chunk before counting it here

// 3. the last digit's decision gives the K-th candidate's key k*, the ties
//    taken and the budget.  Then the ordered compaction: the candidates above
//    k*, then the r lowest-index ties; the slots past the budget become -1.
//    Thread t takes the kPer consecutive candidates c0 + kPer t .., so one
//    block scan of the threads' (above, tie) counts places every candidate:
//    a candidate's slot is the number of chosen candidates before it, i.e.
//    the candidates above k* before it plus min(ties before it, r).  Each
//    chunk publishes its two counts in one atomic word and adds those of the
//    chunks before it (a chunk whose word has not appeared after kSpinLimit
//    polls is counted from its scores instead).  The chunk's slots are filled
//    in LDS and leave as one contiguous run.
__global__ __launch_bounds__(kSelThreads) void sel_write_kernel(SelArgs a) {
  __shared__ int sh[kSelWaves];
  __shared__ uint32_t shk[kSelWaves];
  __shared__ int wsum[2][kSelWaves];
  __shared__ Dec shd;
  __shared__ int32_t stage[kSelChunk];
  __shared__ uint32_t hsc[kBins];
  __shared__ unsigned long long hsm[kBins];
  const int r = blockIdx.y, q = blockIdx.x, c0 = q * kSelChunk;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const RowRef rr = row_ref(a, r);
  const unsigned long long* st = a.state + (size_t)kSelStateWords * r;
  // the chunk's scores arrive coalesced (candidate c0 + kSelThreads j + t in thread
  // t) and are moved through LDS to thread t's own run c0 + kPer t ..: the
  // element of run T at place J sits in slot kPer T + (J ^ (T >> 2)), which
  // keeps both the writes and the reads free of bank conflicts
  const int cb = c0 + kPer * tid;  // this thread's first candidate
  float v[kPer];
  {
    float lv[kPer];
    load_chunk(rr, a.n, c0, lv);
    float* tr = reinterpret_cast<float*>(stage);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = kSelThreads * j + tid, T = e / kPer, J = e % kPer;
      tr[kPer * T + (J ^ ((T >> 2) & (kPer - 1)))] = lv[j];
    }
  }
  Pre f;
  prefetch(a, r, kPasses - 1, f);
  stage_hist(f, hsc, hsm);
  const float mx = row_max(f, shk);  // its barrier also completes the transpose and the staging
  {
    const float* tr = reinterpret_cast<const float*>(stage);
#pragma unroll
    for (int j = 0; j < kPer; ++j) v[j] = tr[kPer * tid + (j ^ ((tid >> 2) & (kPer - 1)))];
  }
  const Dec d = decide(a, r, kPasses - 1, f, hsc, hsm, &shd);
  const uint32_t kstar = (uint32_t)d.prefix;
  // ties needed: every tie has the same mass u*, so it is a division
  unsigned long long T, cap;
  target_of(a, f.U, f.above, r, T, cap);
  unsigned long long ntie = cap - d.cnt_above;
  const unsigned long long ustar = d.bcnt ? d.bmass / d.bcnt : 0ull;
  if (ustar > 0ull) ntie = min(ntie, (T - d.mass_above + ustar - 1ull) / ustar);
  ntie = min(ntie, d.bcnt);
  const long long ties = (long long)ntie;
  const int K = (int)(d.cnt_above + ntie);
  if (q == 0 && tid == 0) *rr.count = K;
  // per-candidate class: 2 above k*, 1 tie, 0 not chosen in any case
  uint32_t cls = 0u;
  int ns = 0, nt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const float s = v[j];
    if (s - mx >= -32.0f) {
      const uint32_t k = order_key(s);
      const uint32_t c = k > kstar ? 2u : (k == kstar ? 1u : 0u);
      cls |= c << (2 * j);
      ns += c == 2u ? 1 : 0;
      nt += c == 1u ? 1 : 0;
    }
  }
  // exclusive scan of (ns, nt) over the block
  const int xs = wave_scan<64>(ns), xt = wave_scan<64>(nt);
  if (lane == 63) {
    wsum[0][wv] = xs;
    wsum[1][wv] = xt;
  }
  __syncthreads();  // also: every thread has read its run, so `stage` is free
  int bs = 0, bt = 0, chunk_s = 0, chunk_t = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    bs += w < wv ? wsum[0][w] : 0;
    bt += w < wv ? wsum[1][w] : 0;
    chunk_s += wsum[0][w];
    chunk_t += wsum[1][w];
  }
  unsigned long long* slots = a.slot + (size_t)r * a.chunks;
  if (tid == 0)
    __hip_atomic_store(&slots[q], kSlotValid | ((unsigned long long)chunk_t << 32) | (unsigned)chunk_s,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the counts of the chunks before this one
  int sb = 0, tb = 0;
  for (int i = tid; i < q; i += kSelThreads) {
    unsigned long long w = 0ull;
    for (int it = 0; it < kSpinLimit; ++it) {
      w = __hip_atomic_load(&slots[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (w & kSlotValid) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (w & kSlotValid) {
      sb += (int)(w & 0xffffffffull);
      tb += (int)((w >> 32) & 0x7fffffffull);
    } else {
      for (int c = i * kSelChunk; c < min((i + 1) * kSelChunk, a.n); ++c) {
        float s = load_score(rr.row, a.n, rr.kind, c);
        s = s == 0.0f ? 0.0f : s;
        if (!(s - mx >= -32.0f)) continue;
        const uint32_t k = order_key(s);
        sb += k > kstar ? 1 : 0;
        tb += k == kstar ? 1 : 0;
      }
    }
  }
  const int strict_chunk = block_reduce(sb, [](int x, int y) { return x + y; }, sh);
  const int tie_chunk = block_reduce(tb, [](int x, int y) { return x + y; }, sh);
  // chosen candidates of earlier chunks, and of this chunk in all
  const long long first = strict_chunk + min((long long)tie_chunk, ties);
  const long long taken = strict_chunk + chunk_s + min((long long)(tie_chunk + chunk_t), ties) - first;
  long long sc = strict_chunk + bs + xs - ns, tc = tie_chunk + bt + xt - nt;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t c = (cls >> (2 * j)) & 3u;
    if (c == 2u) {
      stage[(int)(sc + min(tc, ties) - first)] = cb + j;
      ++sc;
    } else if (c == 1u) {
      if (tc < ties) stage[(int)(sc + tc - first)] = cb + j;
      ++tc;
    }
  }
  __syncthreads();
  int32_t* out = rr.idx;
  for (int i = tid; i < (int)taken; i += kSelThreads)
    if (first + i < rr.cap) out[first + i] = stage[i];
  // this chunk's share of the unused slots
  const int spare = rr.cap - K;
  if (spare > 0) {
    const int per = (spare + a.chunks - 1) / a.chunks;
    const int lo = K + q * per, hi = min(K + (q + 1) * per, rr.cap);
    for (int t = lo + tid; t < hi; t += kSelThreads) out[t] = -1;
  }
}

}  // namespace

hipError_t launch_select_sides(const SelSide* sides, int nsides, int heads, int n, double mass,
                               unsigned long long thresh, void* ws, hipStream_t stream) {
  const int rows = nsides * heads;
  const SelectWsLayout L(rows, n);
  char* base = static_cast<char*>(ws);
  SelArgs a;
  a.side[0] = sides[0];
  a.side[1] = nsides > 1 ? sides[1] : sides[0];
  a.hk = heads;
  a.n = n;
  a.chunks = L.chunks;
  a.mass = mass;
  a.thresh = thresh;
  a.cmax = reinterpret_cast<uint32_t*>(base + L.off_cmax);
  a.state = reinterpret_cast<unsigned long long*>(base + L.off_state);
  a.hcnt = reinterpret_cast<uint32_t*>(base + L.off_hcnt);
  a.hmass = reinterpret_cast<unsigned long long*>(base + L.off_hmass);
  a.slot = reinterpret_cast<unsigned long long*>(base + L.off_slot);
  const dim3 chunks((unsigned)L.chunks, (unsigned)rows);
  hipLaunchKernelGGL(sel_max_kernel, chunks, dim3(kSelThreads), 0, stream, a);
  for (int p = 0; p < kPasses; ++p)
    hipLaunchKernelGGL(sel_hist_kernel, chunks, dim3(kSelThreads), 0, stream, a, p);
  hipLaunchKernelGGL(sel_write_kernel, chunks, dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_select(const float* logit, int heads, int n, int kind, double mass,
                         unsigned long long thresh, int cap, int32_t* idx, int32_t* count, void* ws,
                         hipStream_t stream) {
  const SelSide side{logit, idx, count, kind, cap};
  return launch_select_sides(&side, 1, heads, n, mass, thresh, ws, stream);
}

}  // namespace vs
