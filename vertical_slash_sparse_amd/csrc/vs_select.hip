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
// 8-bit digit, so no element is ever sorted:
//   1. m = max score; u_c = quantised mass of score_c - m (exact integer);
//      U = sum u; T = ceil(mass * U).
//   2. Only scores within 32 of the maximum can be chosen (everything else
//      has u = 0 and sorts after the element that completes T), so digits are
//      taken over the key range of those candidates only.
//   3. Digit by digit from the top, the bucket holding the K-th element in
//      (score descending, index ascending) order is the first whose running
//      mass reaches T or whose running count reaches cap.
//   4. Equal scores have equal u, so the number r of tied elements needed is
//      a division; they are the r lowest indices of the tie.
//   5. An ordered compaction writes the chosen candidates ascending.
// Every pass over the candidates is spread over workgroups of kSelChunk
// candidates (a few hundred workgroups at n = 128K), joined by integer
// atomics in the workspace and a one-block decision per head between passes;
// integer sums are order-free, so the result does not depend on scheduling.
// The same chain serves FlashPrefill's max-based dynamic threshold
// (FlashPrefill summary, Spanish page, section 2.B): keep the candidates whose
// softmax score is at least alpha times the largest, i.e. u >= ceil(alpha *
// 2^32) (the maximum has u = 2^32), at most cap of them in the same order;
// there the budget is that count and no mass target applies.
// The launches form a fixed chain of nine kernels plus two per digit pass
// (at most four); passes the key range does not need return at once.
// The mass arithmetic follows a fixed specification so the budget is an
// exact integer decision: exp is Cody and Waite's range reduction with a
// two-piece ln 2 (W. J. Cody, W. Waite, 1980) and the degree-7 Taylor
// polynomial by explicit fused multiply-adds in fp32; nothing else is fused.
#include "vs_common.h"
#include "vs_internal.h"

#pragma clang fp contract(off)

namespace vs {

namespace {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kMaxPasses = 4;

// per-head decision state (unsigned 64-bit words in the workspace)
enum : int {
  kStMaxKey = 0,   // order key of the maximum score
  kStKmin,         // smallest candidate key
  kStU,            // sum of quantised masses
  kStCand,         // number of candidates
  kStT,            // mass target
  kStPasses,       // digit passes needed
  kStPrefix,       // digits of (key - kmin) fixed so far
  kStMassAbove,    // mass of candidates strictly above the current bucket
  kStCntAbove,     // their number
  kStBucketCnt,    // candidates in the bucket holding the K-th
  kStBucketMass,   // their mass
  kStR,            // ties taken
  kStK,            // budget
  kStCap,          // candidates the selection may take
  kStAbove         // candidates at or above the threshold (threshold mode)
};

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
  uint32_t* key;
  uint64_t* um;
  unsigned long long* state;  // [rows][16]
  uint32_t* hcnt;             // [rows][2][256]
  unsigned long long* hmass;  // [rows][2][256]
  int32_t* cc;                // [rows][chunks][4]: strict, ties, strict before, ties before
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

__global__ __launch_bounds__(kSelThreads) void sel_init_kernel(SelArgs a) {
  const int h = blockIdx.x, tid = threadIdx.x;
  unsigned long long* st = a.state + 16 * (size_t)h;
  if (tid < 16) st[tid] = tid == kStKmin ? 0xffffffffull : 0ull;
  for (int i = tid; i < 512; i += kSelThreads) {
    a.hcnt[512 * (size_t)h + i] = 0u;
    a.hmass[512 * (size_t)h + i] = 0ull;
  }
}

// 1a. maximum score, as its order key
__global__ __launch_bounds__(kSelThreads) void sel_max_kernel(SelArgs a) {
  __shared__ uint32_t sh[kSelWaves];
  const int h = blockIdx.y, c0 = blockIdx.x * kSelChunk;
  const RowRef rr = row_ref(a, h);
  uint32_t km = 0u;
  for (int c = c0 + threadIdx.x; c < min(c0 + kSelChunk, a.n); c += kSelThreads)
    km = max(km, order_key(load_score(rr.row, a.n, rr.kind, c)));
  km = block_reduce(km, [](uint32_t x, uint32_t y) { return max(x, y); }, sh);
  if (threadIdx.x == 0) atomicMax(&a.state[16 * (size_t)h + kStMaxKey], (unsigned long long)km);
}

// 1b. quantised masses, keys, U, candidate count and the smallest candidate key
__global__ __launch_bounds__(kSelThreads) void sel_mass_kernel(SelArgs a) {
  __shared__ unsigned long long shu[kSelWaves];
  __shared__ uint32_t shk[kSelWaves];
  const int h = blockIdx.y, c0 = blockIdx.x * kSelChunk;
  const RowRef rr = row_ref(a, h);
  unsigned long long* st = a.state + 16 * (size_t)h;
  const float mx = key_score((uint32_t)st[kStMaxKey]);
  unsigned long long usum = 0, ncand = 0, nabove = 0;
  uint32_t kmin = 0xffffffffu;
  for (int c = c0 + threadIdx.x; c < min(c0 + kSelChunk, a.n); c += kSelThreads) {
    float s = load_score(rr.row, a.n, rr.kind, c);
    if (s == 0.0f) s = 0.0f;
    const float x = s - mx;
    const bool cand = x >= -32.0f;
    const uint64_t u = spec_mass(x);
    const uint32_t k = order_key(s);
    a.key[(size_t)h * a.n + c] = cand ? k : 0u;
    a.um[(size_t)h * a.n + c] = u;
    usum += u;
    ncand += cand ? 1ull : 0ull;
    nabove += (a.thresh && u >= a.thresh) ? 1ull : 0ull;
    if (cand) kmin = min(kmin, k);
  }
  usum = block_reduce(usum, [](unsigned long long x, unsigned long long y) { return x + y; }, shu);
  ncand = block_reduce(ncand, [](unsigned long long x, unsigned long long y) { return x + y; }, shu);
  nabove = block_reduce(nabove, [](unsigned long long x, unsigned long long y) { return x + y; }, shu);
  kmin = block_reduce(kmin, [](uint32_t x, uint32_t y) { return min(x, y); }, shk);
  if (threadIdx.x == 0) {
    atomicAdd(&st[kStU], usum);
    atomicAdd(&st[kStCand], ncand);
    atomicAdd(&st[kStAbove], nabove);
    atomicMin(&st[kStKmin], (unsigned long long)kmin);
  }
}

// 1c. the target and the digit passes the candidates' key range needs
__global__ void sel_prep_kernel(SelArgs a) {
  const int h = blockIdx.x;
  unsigned long long* st = a.state + 16 * (size_t)h;
  if (threadIdx.x != 0) return;
  const unsigned long long U = st[kStU];
  if (a.thresh) {
    // threshold mode: the budget is the count at or above the threshold; no
    // mass target can stop the walk first (T exceeds the total mass)
    st[kStT] = U + 1ull;
    st[kStCap] = min((unsigned long long)row_ref(a, h).cap, st[kStAbove]);
  } else {
    st[kStT] = (unsigned long long)__builtin_ceil(a.mass * (double)U);
    st[kStCap] = (unsigned long long)row_ref(a, h).cap;
  }
  const uint32_t kmin = (uint32_t)st[kStKmin], kmax = (uint32_t)st[kStMaxKey];
  const uint32_t range = kmax - kmin;
  const int nbits = range ? 32 - __builtin_clz(range) : 0;
  const int npass = (nbits + 7) / 8;
  st[kStPasses] = (unsigned long long)npass;
  st[kStPrefix] = 0ull;
  st[kStMassAbove] = 0ull;
  st[kStCntAbove] = 0ull;
  // with one distinct candidate score every candidate is a tie at kmin
  st[kStBucketCnt] = npass == 0 ? st[kStCand] : 0ull;
  st[kStBucketMass] = npass == 0 ? U : 0ull;
}

// 2-3a. digit histogram (counts and masses) of the candidates that match
//       the fixed digits
__global__ __launch_bounds__(kSelThreads) void sel_hist_kernel(SelArgs a, int pass) {
  __shared__ uint32_t lc[256];
  __shared__ unsigned long long lm[256];
  const int h = blockIdx.y, c0 = blockIdx.x * kSelChunk;
  const unsigned long long* st = a.state + 16 * (size_t)h;
  const int npass = (int)st[kStPasses];
  if (pass >= npass) return;
  const int shift = 8 * (npass - 1 - pass);
  const uint32_t kmin = (uint32_t)st[kStKmin];
  const uint64_t prefix = st[kStPrefix];
  const uint64_t hi_mask = ~((1ull << (shift + 8)) - 1ull);
  for (int i = threadIdx.x; i < 256; i += kSelThreads) {
    lc[i] = 0u;
    lm[i] = 0ull;
  }
  __syncthreads();
  for (int c = c0 + threadIdx.x; c < min(c0 + kSelChunk, a.n); c += kSelThreads) {
    const uint32_t k = a.key[(size_t)h * a.n + c];
    if (k < kmin || k == 0u) continue;
    const uint64_t rel = (uint64_t)(k - kmin);
    if ((rel & hi_mask) != (prefix & hi_mask)) continue;
    const int dg = (int)((rel >> shift) & 255u);
    atomicAdd(&lc[dg], 1u);
    atomicAdd(&lm[dg], (unsigned long long)a.um[(size_t)h * a.n + c]);
  }
  __syncthreads();
  const int par = pass & 1;
  for (int i = threadIdx.x; i < 256; i += kSelThreads)
    if (lc[i]) {
      atomicAdd(&a.hcnt[(512 * (size_t)h) + 256 * par + i], lc[i]);
      atomicAdd(&a.hmass[(512 * (size_t)h) + 256 * par + i], lm[i]);
    }
}

// 2-3b. the bucket holding the K-th candidate; clears the other histogram
__global__ __launch_bounds__(64) void sel_decide_kernel(SelArgs a, int pass) {
  const int h = blockIdx.x, lane = threadIdx.x;
  unsigned long long* st = a.state + 16 * (size_t)h;
  const int npass = (int)st[kStPasses];
  if (pass >= npass) return;
  const int shift = 8 * (npass - 1 - pass);
  const int par = pass & 1;
  const uint32_t* hc = a.hcnt + 512 * (size_t)h + 256 * par;
  const unsigned long long* hm = a.hmass + 512 * (size_t)h + 256 * par;
  const unsigned long long T = st[kStT], cap = st[kStCap];
  const unsigned long long mass_above = st[kStMassAbove], cnt_above = st[kStCntAbove];
  const uint64_t prefix = st[kStPrefix];
  // lane l owns digits 255-4l .. 252-4l (descending)
  unsigned long long lc = 0, lm = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    lc += hc[255 - 4 * lane - q];
    lm += hm[255 - 4 * lane - q];
  }
  unsigned long long sc = lc, sm = lm;  // inclusive scan over lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long yc = __shfl_up(sc, o, 64), ym = __shfl_up(sm, o, 64);
    if (lane >= o) {
      sc += yc;
      sm += ym;
    }
  }
  const unsigned long long ec = sc - lc, em = sm - lm;  // before this lane
  const bool hit = (mass_above + sm >= T) || (cnt_above + sc >= cap);
  const uint64_t hb = __builtin_amdgcn_ballot_w64(hit);
  const int first = hb ? __builtin_ctzll(hb) : 63;
  if (lane == first) {
    unsigned long long rc = ec, rm = em;
    int dsel = 255 - 4 * lane - 3;
    for (int q = 0; q < 4; ++q) {
      const int dg = 255 - 4 * lane - q;
      const unsigned long long bc = hc[dg], bm = hm[dg];
      if (mass_above + rm + bm >= T || cnt_above + rc + bc >= cap) {
        dsel = dg;
        break;
      }
      rc += bc;
      rm += bm;
    }
    st[kStPrefix] = prefix | ((uint64_t)dsel << shift);
    st[kStMassAbove] = mass_above + rm;
    st[kStCntAbove] = cnt_above + rc;
    st[kStBucketCnt] = hc[dsel];
    st[kStBucketMass] = hm[dsel];
  }
  // the histogram the next pass fills
  for (int i = lane; i < 256; i += 64) {
    a.hcnt[512 * (size_t)h + 256 * (par ^ 1) + i] = 0u;
    a.hmass[512 * (size_t)h + 256 * (par ^ 1) + i] = 0ull;
  }
}

// 4a. per chunk: candidates strictly above the K-th key, and ties with it
__global__ __launch_bounds__(kSelThreads) void sel_count_kernel(SelArgs a) {
  __shared__ int sh[kSelWaves];
  const int h = blockIdx.y, q = blockIdx.x, c0 = q * kSelChunk;
  const unsigned long long* st = a.state + 16 * (size_t)h;
  const uint32_t kstar = (uint32_t)st[kStKmin] + (uint32_t)st[kStPrefix];
  int ns = 0, nt = 0;
  for (int c = c0 + threadIdx.x; c < min(c0 + kSelChunk, a.n); c += kSelThreads) {
    const uint32_t k = a.key[(size_t)h * a.n + c];
    ns += (k != 0u && k > kstar) ? 1 : 0;
    nt += (k != 0u && k == kstar) ? 1 : 0;
  }
  ns = block_reduce(ns, [](int x, int y) { return x + y; }, sh);
  nt = block_reduce(nt, [](int x, int y) { return x + y; }, sh);
  if (threadIdx.x == 0) {
    int32_t* cc = a.cc + 4 * ((size_t)h * a.chunks + q);
    cc[0] = ns;
    cc[1] = nt;
  }
}

// 4b. ties needed, the budget, and each chunk's place in the output
__global__ __launch_bounds__(kSelThreads) void sel_scan_kernel(SelArgs a) {
  __shared__ int sh[kSelWaves + 1];
  const int h = blockIdx.x;
  unsigned long long* st = a.state + 16 * (size_t)h;
  const unsigned long long T = st[kStT], mass_above = st[kStMassAbove], cnt_above = st[kStCntAbove];
  const unsigned long long bucket_cnt = st[kStBucketCnt], bucket_mass = st[kStBucketMass];
  unsigned long long r = st[kStCap] - cnt_above;
  const unsigned long long ustar = bucket_cnt ? bucket_mass / bucket_cnt : 0ull;
  if (ustar > 0ull) {
    const unsigned long long need = (T - mass_above + ustar - 1ull) / ustar;
    r = min(r, need);
  }
  r = min(r, bucket_cnt);
  const int K = (int)(cnt_above + r);
  // running totals over chunks, in chunk order
  int strict_before = 0, tie_before = 0;
  for (int q0 = 0; q0 < a.chunks; q0 += kSelThreads) {
    const int q = q0 + threadIdx.x;
    int32_t* cc = a.cc + 4 * ((size_t)h * a.chunks + (q < a.chunks ? q : 0));
    const int ns = q < a.chunks ? cc[0] : 0, nt = q < a.chunks ? cc[1] : 0;
    int tot_s, tot_t;
    // exclusive scans via two block counts of unary flags would be wasteful;
    // a shared-memory scan of the two values
    int xs = ns, xt = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int ys = __shfl_up(xs, o, 64), yt = __shfl_up(xt, o, 64);
      if ((threadIdx.x & 63) >= o) {
        xs += ys;
        xt += yt;
      }
    }
    __shared__ int ws[kSelWaves], wt[kSelWaves];
    if ((threadIdx.x & 63) == 63) {
      ws[threadIdx.x >> 6] = xs;
      wt[threadIdx.x >> 6] = xt;
    }
    __syncthreads();
    int bs = 0, bt = 0;
    tot_s = 0;
    tot_t = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      if (w < (threadIdx.x >> 6)) {
        bs += ws[w];
        bt += wt[w];
      }
      tot_s += ws[w];
      tot_t += wt[w];
    }
    __syncthreads();
    if (q < a.chunks) {
      cc[2] = strict_before + bs + xs - ns;
      cc[3] = tie_before + bt + xt - nt;
    }
    strict_before += tot_s;
    tie_before += tot_t;
  }
  (void)sh;
  if (threadIdx.x == 0) {
    st[kStR] = r;
    st[kStK] = (unsigned long long)K;
    *row_ref(a, h).count = K;
  }
}

// 5. ordered compaction: strictly better keys, then the r lowest-index ties;
//    the slots past the budget become -1
__global__ __launch_bounds__(kSelThreads) void sel_write_kernel(SelArgs a) {
  __shared__ int sh[kSelWaves];
  const int h = blockIdx.y, q = blockIdx.x, c0 = q * kSelChunk;
  const unsigned long long* st = a.state + 16 * (size_t)h;
  const uint32_t kstar = (uint32_t)st[kStKmin] + (uint32_t)st[kStPrefix];
  const long long r = (long long)st[kStR];
  const int K = (int)st[kStK];
  const int32_t* cc = a.cc + 4 * ((size_t)h * a.chunks + q);
  const int strict_before = cc[2], tie_before = cc[3];
  // chosen before this chunk: all strict ones, and the ties among the first r
  const long long ties_taken_before = min((long long)tie_before, r);
  int written = strict_before + (int)ties_taken_before;
  int ties_seen = tie_before;
  const RowRef rr = row_ref(a, h);
  int32_t* out = rr.idx;
  for (int base = c0; base < min(c0 + kSelChunk, a.n); base += kSelThreads) {
    const int c = base + threadIdx.x;
    const bool in = c < min(c0 + kSelChunk, a.n);
    const uint32_t k = in ? a.key[(size_t)h * a.n + c] : 0u;
    const bool strict = in && k != 0u && k > kstar;
    const bool tie = in && k != 0u && k == kstar;
    int tie_total;
    const int tie_rank = ties_seen + block_count(tie, &tie_total, sh);
    const bool take = strict || (tie && (long long)tie_rank < r);
    int take_total;
    const int pos = written + block_count(take, &take_total, sh);
    if (take && pos < rr.cap) out[pos] = c;
    ties_seen += tie_total;
    written += take_total;
  }
  // this chunk's share of the unused slots
  const int spare = rr.cap - K;
  if (spare > 0) {
    const int per = (spare + a.chunks - 1) / a.chunks;
    const int lo = K + q * per, hi = min(K + (q + 1) * per, rr.cap);
    for (int t = lo + threadIdx.x; t < hi; t += kSelThreads) out[t] = -1;
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
  a.key = reinterpret_cast<uint32_t*>(base + L.off_key);
  a.um = reinterpret_cast<uint64_t*>(base + L.off_mass);
  a.state = reinterpret_cast<unsigned long long*>(base + L.off_state);
  a.hcnt = reinterpret_cast<uint32_t*>(base + L.off_hcnt);
  a.hmass = reinterpret_cast<unsigned long long*>(base + L.off_hmass);
  a.cc = reinterpret_cast<int32_t*>(base + L.off_cc);
  const unsigned nrow = (unsigned)rows;
  const dim3 chunks((unsigned)L.chunks, nrow);
  hipLaunchKernelGGL(sel_init_kernel, dim3(nrow), dim3(kSelThreads), 0, stream, a);
  hipLaunchKernelGGL(sel_max_kernel, chunks, dim3(kSelThreads), 0, stream, a);
  hipLaunchKernelGGL(sel_mass_kernel, chunks, dim3(kSelThreads), 0, stream, a);
  hipLaunchKernelGGL(sel_prep_kernel, dim3(nrow), dim3(64), 0, stream, a);
  for (int pass = 0; pass < kMaxPasses; ++pass) {
    hipLaunchKernelGGL(sel_hist_kernel, chunks, dim3(kSelThreads), 0, stream, a, pass);
    hipLaunchKernelGGL(sel_decide_kernel, dim3(nrow), dim3(64), 0, stream, a, pass);
  }
  hipLaunchKernelGGL(sel_count_kernel, chunks, dim3(kSelThreads), 0, stream, a);
  hipLaunchKernelGGL(sel_scan_kernel, dim3(nrow), dim3(kSelThreads), 0, stream, a);
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
