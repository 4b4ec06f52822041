// vs_index.hip -- VSIndexer scoring for gfx950.
//
// VSPrefill (gist.science summaries of arXiv 2603.04460, English page,
// Technical Summary section 2, "Key Components 1. VSIndexer"): a
// shared-weight two-layer linear network over concat(K with RoPE, V) with
// separate down-projection heads for vertical and slash importance:
//     h_j = max(0, W1 [k_j | v_j]),   vlog_j = W2[0] . h_j,   slog_j = W2[1] . h_j.
//
// Each position reads 2*d*2 = 512 bytes and costs 2*256*128 + 2*2*128 flops,
// about 128 flop per byte -- under the MI355X ridge (~315 flop/B for bf16
// MFMA against 8 TB/s), so the kernel is HBM-bound and is built to stream:
//  * persistent workgroups; W1 (64 KiB of bf16) is staged into LDS once per
//    workgroup and serves every position it visits;
//  * H^T = W1 X^T on v_mfma_f32_32x32x16_bf16 with W1 rows as the A operand
//    (from LDS) and 32 positions per wave as the B operand, loaded straight
//    from HBM in the operand layout (16 bytes per lane per k-step, the whole
//    512-byte row consumed by two lanes);
//  * the second layer in fp32 on the vector ALUs from the fp32 accumulators,
//    with the two wave halves' partial sums joined by one lane exchange;
//  * the next 32 positions' rows are loaded before the current ones are
//    multiplied, so HBM traffic overlaps the matrix work.
#include "vs_common.h"
#include "vs_internal.h"

namespace vs {

namespace {

constexpr int kIdxD = 128;          // head dim
constexpr int kIdxX = 2 * kIdxD;    // indexer input width
constexpr int kIdxH = 128;          // hidden width
constexpr int kIdxRow = kIdxX + 8;  // padded LDS row of W1 (bf16)
constexpr int kIdxKS = kIdxX / 16;  // k-steps
constexpr int kIdxHT = kIdxH / 32;  // 32-row tiles of H^T

__global__ __launch_bounds__(256) void index_kernel(const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v,
                                                    const uint16_t* __restrict__ w1,
                                                    const uint16_t* __restrict__ w2,
                                                    float* __restrict__ vlog,
                                                    float* __restrict__ slog,
                                                    long long total_rows) {
  __shared__ __align__(16) uint16_t w1_lds[kIdxH * kIdxRow];
  __shared__ __align__(16) float w2_lds[kIdxH * 2];  // [hidden][vertical, slash]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, ql = lane & 31;
  for (int id = tid; id < kIdxH * kIdxX / 8; id += 256) {
    const int r = id / (kIdxX / 8), c8 = id % (kIdxX / 8);
    *reinterpret_cast<u32x4*>(&w1_lds[r * kIdxRow + 8 * c8]) =
        *reinterpret_cast<const u32x4*>(&w1[r * kIdxX + 8 * c8]);
  }
  for (int id = tid; id < kIdxH * 2; id += 256) {
    const int hid = id >> 1, o = id & 1;
    w2_lds[id] = __uint_as_float((uint32_t)w2[o * kIdxH + hid] << 16);
  }
  __syncthreads();

  const long long step = (long long)gridDim.x * 4 * 32;
  long long r0 = ((long long)blockIdx.x * 4 + wave) * 32;

  auto load_rows = [&](long long base, u32x4 (&bx)[kIdxKS]) {
    const long long row = base + ql;
    const long long rr = row < total_rows ? row : (total_rows - 1);
#pragma unroll
    for (int s = 0; s < kIdxKS; ++s) {
      const uint16_t* src = s < kIdxKS / 2 ? k + rr * kIdxD + 16 * s + 8 * half
                                           : v + rr * kIdxD + 16 * (s - kIdxKS / 2) + 8 * half;
      bx[s] = *reinterpret_cast<const u32x4*>(src);
    }
  };

  u32x4 cur[kIdxKS];
  if (r0 < total_rows) load_rows(r0, cur);
  for (; r0 < total_rows; r0 += step) {
    u32x4 nxt[kIdxKS];
    const bool more = r0 + step < total_rows;
    if (more) load_rows(r0 + step, nxt);
    f32x16 acc[kIdxHT];
#pragma unroll
    for (int t = 0; t < kIdxHT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
#pragma unroll
    for (int s = 0; s < kIdxKS; ++s) {
      const bf16x8 b = as_bf16x8(cur[s]);
#pragma unroll
      for (int t = 0; t < kIdxHT; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&w1_lds[(32 * t + ql) * kIdxRow + 16 * s + 8 * half]);
        acc[t] = mfma32(a, b, acc[t]);
      }
    }
    // second layer: this lane holds hidden units 32t + 8a + 4*half + 0..3
    float pv = 0.f, ps = 0.f;
#pragma unroll
    for (int t = 0; t < kIdxHT; ++t)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int h0 = 32 * t + 8 * a + 4 * half;
        const float4 wa = *reinterpret_cast<const float4*>(&w2_lds[2 * h0]);
        const float4 wb = *reinterpret_cast<const float4*>(&w2_lds[2 * h0 + 4]);
        const float x0 = fmaxf(acc[t][4 * a + 0], 0.f), x1 = fmaxf(acc[t][4 * a + 1], 0.f);
        const float x2 = fmaxf(acc[t][4 * a + 2], 0.f), x3 = fmaxf(acc[t][4 * a + 3], 0.f);
        pv = fmaf(x0, wa.x, pv);
        ps = fmaf(x0, wa.y, ps);
        pv = fmaf(x1, wa.z, pv);
        ps = fmaf(x1, wa.w, ps);
        pv = fmaf(x2, wb.x, pv);
        ps = fmaf(x2, wb.y, ps);
        pv = fmaf(x3, wb.z, pv);
        ps = fmaf(x3, wb.w, ps);
      }
    pv += swap_halves(pv);
    ps += swap_halves(ps);
    const long long row = r0 + ql;
    if (half == 0 && row < total_rows) {
      vlog[row] = pv;
      slog[row] = ps;
    }
    if (more) {
#pragma unroll
      for (int s = 0; s < kIdxKS; ++s) cur[s] = nxt[s];
    }
  }
}

}  // namespace

hipError_t launch_index(const void* k, const void* v, int h_kv, int n, const void* w1,
                        const void* w2, float* vlog, float* slog, hipStream_t stream) {
  const long long total = (long long)h_kv * n;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
      cus = c;
  }
  const long long want = (total + 127) / 128;
  const long long grid = want < 2LL * cus ? want : 2LL * cus;
  hipLaunchKernelGGL(index_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w2), vlog,
                     slog, total);
  return hipGetLastError();
}

}  // namespace vs
