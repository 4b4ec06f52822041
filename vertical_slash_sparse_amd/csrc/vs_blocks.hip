// vs_blocks.hip -- FlashPrefill block discovery for gfx950: block-mean keys,
// skeleton-probe block scores and the max-based threshold, written out as a
// per-query-block bitmap of key blocks.
//
// What is computed (FlashPrefill, gist.science summary of arXiv 2603.06199,
// Spanish page, section 2.A "Estrategia de Aproximacion de Bloques" and 2.B
// "Umbralizacion Dinamica Basada en Maximos"): a sparse set of evenly spaced
// probe queries of each query block is scored against the mean key of every
// earlier key block (exp of that score is the geometric mean of the block's
// exponentials, the AM-GM proxy); a block's score is the probes' softmax
// probability of it, averaged over the probes; a query block keeps the key
// blocks scoring at least alpha times its best, and always its own diagonal
// block.  Blocks are 64 positions, the attention kernel's key tile.
//
// Layout on the chip
//  * blk_mean_kernel: one workgroup per (KV head, key block) sums the block's
//    rows in fp32 (each thread one 16-byte column chunk over a strided set of
//    rows, then the row groups meet in LDS) and stores the mean as a bf16
//    pair hi + lo (hi = bf16(mean), lo = bf16(mean - hi)), about 16
//    significant bits, so the matrix cores can take it.
//  * blk_score_kernel: one wave per query block, eight per workgroup.  The
//    wave's 32 probe rows (G heads x skel rows, zero-padded) are one MFMA
//    operand held in registers; the block means pass through LDS in chunks
//    of 32 blocks (hi and lo, 16 KiB at d = 128), brought in once per
//    workgroup by LDS-DMA two stages deep and read by all eight waves, whose
//    query blocks need nearly the same chunks.  Pass 1 runs
//    S^T = Kbar Q^T, so each lane owns one probe and keeps its running max
//    and sum over blocks; passes 2 and 3 run S = Q Kbar^T, so each lane owns
//    one block and adds the probes' normalised probabilities over its
//    elements, keeps the row's largest score and stores every score in a
//    workspace row; pass 3 reads the row back and thresholds it (one fp32
//    product) into mask words through ballots, a word per chunk.  The score
//    rows live in HBM (4 nb^2 bytes per KV head), not LDS, which keeps LDS to
//    the chunk stages (32 KiB), so several workgroups share a CU.
#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

namespace {

constexpr int kBlkWaves = 8;  // query blocks per workgroup
constexpr int kBlkThreads = kBlkWaves * 64;
constexpr float kNegBig = -1.0e30f;

struct BlkParams {
  const uint16_t* q;    // bf16 [hq][n][d]
  const uint16_t* khi;  // bf16 [hkv][nb][d]: mean keys, high part
  const uint16_t* klo;  // low part
  uint32_t* mask;       // [hkv][nb][wpr]
  float* score;         // optional [hkv][nb][nb]
  float* sc;            // workspace [hkv][nb][nb]: pass 2's scores for pass 3
  int n, nb, hkv, group, skel, wpr;
  float c;              // scale * log2(e)
  float alpha;
};

template <int D>
__global__ __launch_bounds__(256) void blk_mean_kernel(const uint16_t* __restrict__ k,
                                                       uint16_t* __restrict__ khi,
                                                       uint16_t* __restrict__ klo, int n, int nb) {
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int RG = 256 / CH;         // row groups
  __shared__ float part[RG][D];
  const int J = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, ch = tid % CH, rg = tid / CH;
  const int j0 = J * kBN;
  const int cnt = min(kBN, n - j0);
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = rg; r < cnt; r += RG) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(k + ((size_t)g * n + j0 + r) * D + 8 * ch);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[2 * e] += bf16_lo(w[e]);
      s[2 * e + 1] += bf16_hi(w[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][8 * ch + e] = s[e];
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
    for (int r = 0; r < RG; ++r) t += part[r][tid];
    const float mean = t / (float)cnt;
    const __bf16 hi = (__bf16)mean;
    const __bf16 lo = (__bf16)(mean - (float)hi);
    const size_t o = ((size_t)g * nb + J) * D + tid;
    khi[o] = __builtin_bit_cast(uint16_t, hi);
    klo[o] = __builtin_bit_cast(uint16_t, lo);
  }
}

// XOR swizzle of the 16-byte chunks of an LDS row of block means, so that
// the 32 lanes reading one chunk of 32 consecutive rows hit distinct banks
template <int D>
__device__ __forceinline__ int blk_swz(int r) {
  if constexpr (D == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

template <int D>
__global__ __launch_bounds__(kBlkThreads) void blk_score_kernel(BlkParams p) {
  constexpr int KS = D / 16;
  constexpr int CH = D / 8;                      // 16-byte chunks per row
  constexpr int ROWB = D * 2;                    // bytes of one mean-key row
  constexpr int PARTB = 32 * ROWB;               // 32 rows of one part (hi or lo)
  constexpr int STB = 2 * PARTB;                 // one LDS stage: hi rows, then lo rows
  constexpr int RPD = 1024 / ROWB;               // rows per 1 KiB DMA
  constexpr int NDMA = STB / 1024 / kBlkWaves;   // DMAs per wave per chunk
  static_assert(NDMA >= 1 && NDMA * kBlkWaves * 1024 == STB, "chunk split");
  __shared__ __align__(16) uint8_t stages[2 * STB];                 // two chunk stages
  __shared__ float st_m[kBlkWaves][32], st_w[kBlkWaves][32];  // per probe: max, weight / sum
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8* const stg = (lds_u8*)stages;

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, ql = lane & 31;
  const int wave = wave_uniform(tid >> 6);
  const int g = blockIdx.x % p.hkv;
  const int nbw = (p.nb + kBlkWaves - 1) / kBlkWaves;
  const int I0 = (nbw - 1 - (int)(blockIdx.x / p.hkv)) * kBlkWaves;  // longest rows first
  const int I = I0 + wave;                      // this wave's query block
  const bool active = I < p.nb;
  const int n = p.n, nb = p.nb;

  // probe slot ql: head ql / skel of the group, row 64 I + (ql % skel) * (64 / skel)
  const int step = kBN / p.skel;
  const int slot_head = ql / p.skel, slot_m = ql % p.skel;
  const int prow = I * kBN + slot_m * step;
  const bool probe = active && slot_head < p.group && prow < n;
  const int rows_in = active ? min(p.skel, (n - I * kBN + step - 1) / step) : 1;
  const float weight = 1.f / (float)(p.group * rows_in);
  // The probes enter with the sign of the scale folded in (every element
  // flips when it is negative), so that logits are products with |c| and a
  // chunk's largest logit is |c| times its largest product.
  const float cpos = fabsf(p.c);
  bf16x8 qf[KS];
  {
    const int h = g * p.group + min(slot_head, p.group - 1);
    const size_t ro = ((size_t)h * n + min(prow, n - 1)) * D;
    const uint32_t qx = p.c < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(p.q + ro + 16 * s + 8 * half);
#pragma unroll
      for (int e = 0; e < 4; ++e) raw[e] ^= qx;
      if (!probe) raw = u32x4{0u, 0u, 0u, 0u};
      qf[s] = as_bf16x8(raw);
    }
  }

  // chunk c = mean keys of blocks 32 c .. 32 c + 31 of head g, hi and lo,
  // brought into stage st by the eight waves (rows past nb arrive as zeros)
  const uint32_t tab_bytes = (uint32_t)((size_t)p.hkv * nb * ROWB);
  const u32x4 whi = buffer_words(p.khi, tab_bytes);
  const u32x4 wlo = buffer_words(p.klo, tab_bytes);
  int dma_part[NDMA], dma_dst[NDMA], dma_row[NDMA], dma_col[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int kib = wave * NDMA + i;               // KiB of the stage this DMA fills
    const int part = kib / (PARTB / 1024), kin = kib % (PARTB / 1024);
    const int r = kin * RPD + lane / CH;
    dma_part[i] = part;
    dma_dst[i] = part * PARTB + kin * 1024;
    dma_row[i] = r;
    dma_col[i] = 16 * ((lane % CH) ^ blk_swz<D>(r));  // LDS slot lane % CH holds this source chunk
  }
  unsigned dma_off[NDMA];
  auto stage = [&](int c, int st) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int J = 32 * c + dma_row[i];
      const unsigned off = J < nb ? (unsigned)(((size_t)g * nb + J) * ROWB) + dma_col[i] : tab_bytes;
      dma16(dma_part[i] ? wlo : whi, (uint32_t)(uintptr_t)(stg + st * STB + dma_dst[i]), off);
      dma_off[i] = off;
    }
  };
  // operand fragment of row ql (block 32 c + ql) in stage st: dims 16 s + 8 half ..
  auto kfrag = [&](int st, int part, int s) -> bf16x8 {
    return *(const __attribute__((address_space(3))) bf16x8*)(
        stg + st * STB + part * PARTB + ql * ROWB + 16 * ((2 * s + half) ^ blk_swz<D>(ql)));
  };
  const int Imax = min(I0 + kBlkWaves - 1, nb - 1);
  const int nch = (Imax + 31) / 32;          // chunks any wave of the workgroup needs
  const int mych = active ? (I + 31) / 32 : 0;  // candidates of this wave: blocks 0 .. I-1

  // run `body(c, st)` over the chunks, two stages deep
  auto sweep = [&](auto&& body) {
    if (nch == 0) return;
    stage(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      const int st = c & 1;
      if (c + 1 < nch) {
        stage(c + 1, st ^ 1);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) asm volatile("" ::"v"(dma_off[i]));
      }
      if (c < mych) body(c, st);
      __builtin_amdgcn_s_waitcnt(0x0070);  // the next chunk has landed; this one is read
      __syncthreads();
    }
  };

  // ---- pass 1: S^T = Kbar Q^T; lane (ql, half) holds probe ql against
  // blocks 32 c + 8 (e / 4) + 4 half + e % 4
  float m2 = kNegBig, l = 0.f;
  sweep([&](int c, int st) {
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma32(kfrag(st, 0, s), qf[s], acc);
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma32(kfrag(st, 1, s), qf[s], acc);
    float mn, add = 0.f;
    if (32 * c + 32 <= I) {
      // every block of the chunk lies below I: no masks
      float a = acc[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) a = fmaxf(a, acc[e]);
      mn = fmaxf(m2, a * cpos);
#pragma unroll
      for (int e = 0; e < 16; ++e) add += __builtin_amdgcn_exp2f(fmaf(acc[e], cpos, -mn));
    } else {
      float mloc = kNegBig;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int J = c * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
        if (J < I) mloc = fmaxf(mloc, acc[e] * cpos);
      }
      mn = fmaxf(m2, mloc);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int J = c * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
        add += J < I ? __builtin_amdgcn_exp2f(fmaf(acc[e], cpos, -mn)) : 0.f;
      }
    }
    l = l * __builtin_amdgcn_exp2f(m2 - mn) + add;
    m2 = mn;
  });
  {
    // the two halves of the wave saw different blocks of the same probe
    const auto sm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m2), __float_as_uint(m2), false, false);
    const auto sl = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    const float ma = __uint_as_float(sm[0]), mb = __uint_as_float(sm[1]);
    const float M = fmaxf(ma, mb);
    const float L = __uint_as_float(sl[0]) * __builtin_amdgcn_exp2f(ma - M) +
                    __uint_as_float(sl[1]) * __builtin_amdgcn_exp2f(mb - M);
    if (half == 0) {
      st_m[wave][ql] = M;
      st_w[wave][ql] = probe && L > 0.f ? weight / L : 0.f;
    }
  }
  __syncthreads();

  // ---- passes 2 and 3: S = Q Kbar^T; lane (ql, half) holds block 32 c + ql
  // against probes 8 (e / 4) + 4 half + e % 4.  Pass 2 finds the row's
  // largest score and stores the scores; pass 3 thresholds the stored values,
  // one chunk of 32 blocks to a mask word.
  float nm[16], wl[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int pr = 8 * (e >> 2) + 4 * half + (e & 3);
    nm[e] = -st_m[wave][pr];
    wl[e] = st_w[wave][pr];
  }
  auto score_of = [&](int st) -> float {
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma32(qf[s], kfrag(st, 0, s), acc);
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma32(qf[s], kfrag(st, 1, s), acc);
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) t = fmaf(__builtin_amdgcn_exp2f(fmaf(acc[e], cpos, nm[e])), wl[e], t);
    return half_sum(t);
  };
  // pass 2 keeps each score in its lane's slot of the workspace row (lanes
  // of the low half; both halves hold the same sum), where pass 3 reads it
  // back in the same lane
  float* const wrow = p.sc + ((size_t)g * nb + (active ? I : 0)) * nb;
  float mx = 0.f;
  sweep([&](int c, int st) {
    const float t = score_of(st);
    const int J = c * 32 + ql;
    if (J < I) mx = fmaxf(mx, t);
    if (half == 0 && J < nb) wrow[J] = t;
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  // threshold: alpha times the row's largest score, one fp32 product
  const float thr = __fmul_rn(p.alpha, mx);
  uint32_t* mrow = p.mask + ((size_t)g * nb + I) * p.wpr;
  float* srow = p.score ? p.score + ((size_t)g * nb + I) * nb : nullptr;
  if (!active) return;
  for (int c = 0; c < mych; ++c) {
    const int J = c * 32 + ql;
    const float t = half == 0 && J < nb ? wrow[J] : 0.f;
    const bool keep = J == I || (J < I && t >= thr);
    const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);  // the mask word takes the low half
    if (lane == 0) mrow[c] = (uint32_t)bal;
    if (srow && half == 0 && J < nb) srow[J] = J < I ? t : 0.f;
  }
  // words past the last chunk: only the diagonal can be set there
  for (int w = mych + lane; w < p.wpr; w += 64) mrow[w] = I / 32 == w ? 1u << (I % 32) : 0u;
  if (srow)
    for (int J = 32 * mych + lane; J < nb; J += 64) srow[J] = 0.f;
}

}  // namespace

size_t block_workspace_bytes(int h_kv, int n, int d) {
  const size_t nb = (size_t)(n + kBN - 1) / kBN;
  return 2 * align_up(sizeof(uint16_t) * (size_t)h_kv * nb * d, 256) +
         align_up(sizeof(float) * (size_t)h_kv * nb * nb, 256);
}

bool block_discover_grid_fits(int h_kv, long long n) {
  const long long nb = (n + kBN - 1) / kBN;
  return (nb + kBlkWaves - 1) / kBlkWaves * h_kv * kBlkThreads < (1LL << 32) && nb * 256 < (1LL << 32);
}

hipError_t launch_block_discover(const void* q, const void* k, int h_q, int h_kv, int n, int d,
                                 float scale, int skel, float alpha, uint32_t* mask, int wpr,
                                 float* score, void* ws, hipStream_t stream) {
  const int nb = (n + kBN - 1) / kBN;
  uint16_t* khi = static_cast<uint16_t*>(ws);
  uint16_t* klo = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) +
                                              align_up(sizeof(uint16_t) * (size_t)h_kv * nb * d, 256));
  const dim3 mg((unsigned)nb, (unsigned)h_kv);
  if (d == 128)
    hipLaunchKernelGGL(blk_mean_kernel<128>, mg, dim3(256), 0, stream, static_cast<const uint16_t*>(k), khi, klo, n, nb);
  else
    hipLaunchKernelGGL(blk_mean_kernel<64>, mg, dim3(256), 0, stream, static_cast<const uint16_t*>(k), khi, klo, n, nb);
  BlkParams prm;
  prm.q = static_cast<const uint16_t*>(q);
  prm.khi = khi;
  prm.klo = klo;
  prm.mask = mask;
  prm.score = score;
  prm.sc = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                    2 * align_up(sizeof(uint16_t) * (size_t)h_kv * nb * d, 256));
  prm.n = n;
  prm.nb = nb;
  prm.hkv = h_kv;
  prm.group = h_q / h_kv;
  prm.skel = skel;
  prm.wpr = wpr;
  prm.c = scale * 1.4426950408889634f;
  prm.alpha = alpha;
  const dim3 sg((unsigned)(((nb + kBlkWaves - 1) / kBlkWaves) * h_kv));
  if (d == 128)
    hipLaunchKernelGGL(blk_score_kernel<128>, sg, dim3(kBlkThreads), 0, stream, prm);
  else
    hipLaunchKernelGGL(blk_score_kernel<64>, sg, dim3(kBlkThreads), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace vs
