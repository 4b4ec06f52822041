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
//   5. One ordered compaction pass writes the chosen candidates ascending.
// The mass arithmetic follows a fixed specification so the budget is an
// exact integer decision: exp is Cody and Waite's range reduction with a
// two-piece ln 2 (W. J. Cody, W. Waite, 1980) and the degree-7 Taylor
// polynomial by explicit fused multiply-adds in fp32; nothing else is fused.
#include "vs_common.h"
#include "vs_internal.h"

#pragma clang fp contract(off)

namespace vs {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

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

__device__ __forceinline__ float load_score(const float* row, int n, int kind, int c) {
  return kind == 0 ? row[c] : row[n - 1 - c];
}

template <typename T, typename Op>
__device__ T wave_reduce(T x, Op op) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = op(x, __shfl_xor(x, o, 64));
  return x;
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

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ logit, int n,
                                                             int kind, double mass, int cap,
                                                             int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ count,
                                                             uint32_t* __restrict__ key_ws,
                                                             uint64_t* __restrict__ mass_ws) {
  __shared__ float shf[kSelWaves];
  __shared__ unsigned long long shu[kSelWaves];
  __shared__ uint32_t shk[kSelWaves];
  __shared__ int shc[kSelWaves + 1];
  __shared__ uint32_t hcnt[256];
  __shared__ unsigned long long hmass[256];
  __shared__ unsigned long long sel_state[4];  // prefix, mass_above, cnt_above, bucket

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int h = blockIdx.x;
  const float* row = logit + (size_t)h * n;
  uint32_t* key = key_ws + (size_t)h * n;
  uint64_t* um = mass_ws + (size_t)h * n;

  // 1a. maximum score
  float mx = -__builtin_inff();
  for (int c = tid; c < n; c += kSelThreads) mx = fmaxf(mx, load_score(row, n, kind, c));
  mx = wave_reduce(mx, [](float a, float b) { return fmaxf(a, b); });
  if (lane == 0) shf[wv] = mx;
  __syncthreads();
  mx = shf[0];
  for (int w = 1; w < kSelWaves; ++w) mx = fmaxf(mx, shf[w]);
  if (mx == 0.0f) mx = 0.0f;

  // 1b. quantised masses, keys, U and the smallest candidate key
  unsigned long long usum = 0;
  uint32_t kmin = 0xffffffffu;
  for (int c = tid; c < n; c += kSelThreads) {
    float s = load_score(row, n, kind, c);
    if (s == 0.0f) s = 0.0f;
    const float x = s - mx;
    const bool cand = x >= -32.0f;
    const uint64_t u = spec_mass(x);
    const uint32_t k = order_key(s);
    key[c] = cand ? k : 0u;
    um[c] = u;
    usum += u;
    if (cand) kmin = min(kmin, k);
  }
  usum = wave_reduce(usum, [](unsigned long long a, unsigned long long b) { return a + b; });
  kmin = wave_reduce(kmin, [](uint32_t a, uint32_t b) { return min(a, b); });
  if (lane == 0) {
    shu[wv] = usum;
    shk[wv] = kmin;
  }
  __syncthreads();
  unsigned long long U = 0;
  kmin = 0xffffffffu;
  for (int w = 0; w < kSelWaves; ++w) {
    U += shu[w];
    kmin = min(kmin, shk[w]);
  }
  const uint32_t kmax = order_key(mx);
  const unsigned long long T = (unsigned long long)__builtin_ceil(mass * (double)U);

  // 2-3. radix select over rel = key - kmin of candidates
  const uint32_t range = kmax - kmin;
  const int nbits = range ? 32 - __builtin_clz(range) : 0;
  const int npass = (nbits + 7) / 8;
  uint64_t prefix = 0;  // determined bits of rel
  unsigned long long mass_above = 0, cnt_above = 0;
  unsigned long long bucket_cnt = 0, bucket_mass = 0;
  if (npass == 0) {
    // every candidate has the same score
    int tot;
    int dummy = 0;
    for (int base = 0; base < n; base += kSelThreads) {
      const int c = base + tid;
      dummy += (c < n && key[c] >= kmin && key[c] != 0u) ? 1 : 0;
    }
    dummy = wave_reduce(dummy, [](int a, int b) { return a + b; });
    if (lane == 0) shc[wv] = dummy;
    __syncthreads();
    tot = 0;
    for (int w = 0; w < kSelWaves; ++w) tot += shc[w];
    __syncthreads();
    bucket_cnt = (unsigned long long)tot;
    bucket_mass = U;
  }
  for (int pass = 0; pass < npass; ++pass) {
    const int shift = 8 * (npass - 1 - pass);
    for (int i = tid; i < 256; i += kSelThreads) {
      hcnt[i] = 0u;
      hmass[i] = 0ull;
    }
    __syncthreads();
    const uint64_t hi_mask = ~((1ull << (shift + 8)) - 1ull);
    for (int c = tid; c < n; c += kSelThreads) {
      const uint32_t k = key[c];
      if (k < kmin || k == 0u) continue;
      const uint64_t rel = (uint64_t)(k - kmin);
      if ((rel & hi_mask) != (prefix & hi_mask)) continue;
      const int dg = (int)((rel >> shift) & 255u);
      atomicAdd(&hcnt[dg], 1u);
      atomicAdd(&hmass[dg], (unsigned long long)um[c]);
    }
    __syncthreads();
    if (wv == 0) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      unsigned long long lc = 0, lm = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lc += hcnt[255 - 4 * lane - q];
        lm += hmass[255 - 4 * lane - q];
      }
      // inclusive scan over lanes
      unsigned long long sc = lc, sm = lm;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long yc = __shfl_up(sc, o, 64), ym = __shfl_up(sm, o, 64);
        if (lane >= o) {
          sc += yc;
          sm += ym;
        }
      }
      const unsigned long long ec = sc - lc, em = sm - lm;  // exclusive, before this lane
      const bool hit = (mass_above + sm >= T) || (cnt_above + sc >= (unsigned long long)cap);
      const uint64_t hb = __builtin_amdgcn_ballot_w64(hit);
      const int first = hb ? __builtin_ctzll(hb) : 63;
      if (lane == first) {
        unsigned long long rc = ec, rm = em;
        int dsel = 255 - 4 * lane - 3;
        for (int q = 0; q < 4; ++q) {
          const int dg = 255 - 4 * lane - q;
          const unsigned long long bc = hcnt[dg], bm = hmass[dg];
          if (mass_above + rm + bm >= T || cnt_above + rc + bc >= (unsigned long long)cap) {
            dsel = dg;
            break;
          }
          rc += bc;
          rm += bm;
        }
        sel_state[0] = prefix | ((uint64_t)dsel << shift);
        sel_state[1] = mass_above + rm;
        sel_state[2] = cnt_above + rc;
        sel_state[3] = (unsigned long long)dsel;
      }
    }
    __syncthreads();
    prefix = sel_state[0];
    mass_above = sel_state[1];
    cnt_above = sel_state[2];
    const int dsel = (int)sel_state[3];
    bucket_cnt = hcnt[dsel];
    bucket_mass = hmass[dsel];
    __syncthreads();
  }
  const uint32_t kstar = kmin + (uint32_t)prefix;

  // 4. how many of the tied elements are needed
  unsigned long long r = (unsigned long long)cap - cnt_above;
  const unsigned long long ustar = bucket_cnt ? bucket_mass / bucket_cnt : 0ull;
  if (ustar > 0ull) {
    const unsigned long long need = (T - mass_above + ustar - 1ull) / ustar;
    r = min(r, need);
  }
  r = min(r, bucket_cnt);
  const int K = (int)(cnt_above + r);

  // 5. ordered compaction: strictly better keys, then the r lowest-index ties
  int32_t* out = idx + (size_t)h * cap;
  int ties_seen = 0, written = 0;
  for (int base = 0; base < n; base += kSelThreads) {
    const int c = base + tid;
    const uint32_t k = c < n ? key[c] : 0u;
    const bool strict = c < n && k != 0u && k > kstar;
    const bool tie = c < n && k != 0u && k == kstar;
    int tie_total;
    const int tie_rank = ties_seen + block_count(tie, &tie_total, shc);
    const bool take = strict || (tie && (unsigned long long)tie_rank < r);
    int take_total;
    const int pos = written + block_count(take, &take_total, shc);
    if (take && pos < cap) out[pos] = c;
    ties_seen += tie_total;
    written += take_total;
  }
  for (int t = K + tid; t < cap; t += kSelThreads) out[t] = -1;
  if (tid == 0) count[h] = K;
}

}  // namespace

hipError_t launch_select(const float* logit, int heads, int n, int kind, double mass, int cap,
                         int32_t* idx, int32_t* count, void* ws, hipStream_t stream) {
  const SelectWsLayout L(heads, n);
  char* base = static_cast<char*>(ws);
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)heads), dim3(kSelThreads), 0, stream, logit, n,
                     kind, mass, cap, idx, count, reinterpret_cast<uint32_t*>(base + L.off_key),
                     reinterpret_cast<uint64_t*>(base + L.off_mass));
  return hipGetLastError();
}

}  // namespace vs
