// fa_quant.hip -- block quantisation of attention inputs to OCP e4m3 for gfx950, with
// optional incoherent processing, and its C ABI.
//
// The abstract of "FlashAttention-3: Fast and Accurate Attention with Asynchrony and
// Low-precision" names block quantisation and incoherent processing as the two parts of
// its FP8 mode. Here, per (batch, head) and per slab of FA_FP8_BLOCK_ROWS = 64 consecutive
// sequence positions (the key-tile height of the attention kernels):
//   * optional rotation of each row: x <- (x * s) H, s the caller's random signs and H
//     the Sylvester-Hadamard matrix (entries +-1, H H^T = d I), as an unnormalised fast
//     Walsh-Hadamard transform in float32 (butterfly stages h = 1, 2, ..., d/2), which
//     spreads a few large elements over the whole row;
//   * one power-of-two scale per slab, 2^e with e the smallest integer that brings the
//     slab's largest magnitude to at most 448, floored at -127 (0 for a zero slab), stored
//     as an E8M0 byte e + 127 -- the shared-exponent form the gfx950 scaled MFMA and
//     conversion instructions apply exactly;
//   * codes = e4m3 round-to-nearest-even of x * 2^-e (exact scaling).
//
// gfx950 mapping: HBM-bound (2 bytes in, 1 byte out per element). One 256-thread
// workgroup per slab; a row of d elements is held by d/8 consecutive lanes, 8 elements
// (one 16-byte load) each, so loads and stores are contiguous per row. The transform's
// stages h < 8 run inside a lane, the others between lanes l and l ^ (h/8). The slab's
// maximum is reduced over the wavefront by butterfly shuffles and over the four
// wavefronts through LDS; values stay in registers between the two passes.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fa.h"
#include "fa_env.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRows = FA_FP8_BLOCK_ROWS;   // rows per slab
constexpr int kThreads = 256;

struct QuantArgs {
  const void* x;
  const float* signs;    // d floats or null
  uint8_t* codes;
  uint8_t* scales;
  int N, Hx, nb;         // nb = ceil(N / kRows)
};

__device__ __forceinline__ float bf16_to_f32(unsigned short h) { return __uint_as_float((unsigned)h << 16); }
__device__ __forceinline__ float f16_to_f32(unsigned short h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// exponent of the slab scale: smallest e with amax * 2^-e <= 448, floored at -127
__device__ __forceinline__ int slab_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e2;
  (void)frexpf(amax, &e2);                 // amax in [2^(e2-1), 2^e2)
  const int E = e2 - 1;
  int e = ldexpf(amax, 8 - E) <= 448.0f ? E - 8 : E - 7;
  return e < -127 ? -127 : e;
}

template <int D, bool BF16, bool ROTATE>
__global__ __launch_bounds__(kThreads) void quantize_e4m3_block_kernel(QuantArgs a) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerPass = kThreads / kLanesPerRow;
  constexpr int kPasses = kRows / kRowsPerPass;
  static_assert(kPasses * kRowsPerPass == kRows, "slab rows split evenly over passes");

  const int tid = threadIdx.x;
  const int slab = blockIdx.x;             // (b, hx, blk), blk fastest
  const int blk = slab % a.nb;
  const int bh = slab / a.nb;              // b * Hx + hx
  const int hx = bh % a.Hx, b = bh / a.Hx;
  const int chunk = tid % kLanesPerRow;    // elements 8*chunk .. 8*chunk+7 of a row
  const int r_in_pass = tid / kLanesPerRow;
  const int r0 = blk * kRows;
  const size_t row_stride = (size_t)a.Hx * D;
  const size_t base = ((size_t)b * a.N) * row_stride + (size_t)hx * D + (size_t)chunk * 8;

  float sg[8];
  if constexpr (ROTATE) {
    const float4 s0 = *(const float4*)(a.signs + chunk * 8);
    const float4 s1 = *(const float4*)(a.signs + chunk * 8 + 4);
    sg[0] = s0.x; sg[1] = s0.y; sg[2] = s0.z; sg[3] = s0.w;
    sg[4] = s1.x; sg[5] = s1.y; sg[6] = s1.z; sg[7] = s1.w;
  }

  float v[kPasses][8];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int row = r0 + p * kRowsPerPass + r_in_pass;
    const bool live = row < a.N;                         // uniform per row group
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (live) raw = *(const u32x4*)((const uint16_t*)a.x + base + (size_t)row * row_stride);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned short h = (unsigned short)(raw[i >> 1] >> (16 * (i & 1)));
      v[p][i] = BF16 ? bf16_to_f32(h) : f16_to_f32(h);
    }
    if constexpr (ROTATE) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[p][i] *= sg[i];
      // stages h = 1, 2, 4 inside the lane
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if ((i & h) == 0) {
            const float x0 = v[p][i], x1 = v[p][i + h];
            v[p][i] = x0 + x1;
            v[p][i + h] = x0 - x1;
          }
      // stages h = 8, 16, ..., D/2 between lanes: partner lane holds element j ^ h
#pragma unroll
      for (int m = 1; m < kLanesPerRow; m <<= 1) {
        const bool upper = (chunk & m) != 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float other = __shfl_xor(v[p][i], m, 64);
          v[p][i] = upper ? other - v[p][i] : v[p][i] + other;
        }
      }
    }
    if (live)
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[p][i]));
  }

  // slab maximum: butterfly over the wavefront, then over the four wavefronts
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  __shared__ float wmax[kThreads / 64];
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int e = slab_exponent(amax);
  if (tid == 0) a.scales[(size_t)bh * a.nb + blk] = (uint8_t)(e + 127);

#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int row = r0 + p * kRowsPerPass + r_in_pass;
    if (row >= a.N) continue;
    u32x2 out;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = fminf(fmaxf(ldexpf(v[p][4 * w + i], -e), -448.0f), 448.0f);
      int c = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);   // round to nearest even
      c = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], c, true);
      out[w] = (unsigned)c;
    }
    *(u32x2*)(a.codes + base + (size_t)row * row_stride) = out;   // same layout, 1 byte per element
  }
}

template <int D, bool BF16, bool ROTATE>
fa_status launch_quant(const QuantArgs& args, int grid, hipStream_t s) {
  fa_env::log_launch("quantize_e4m3_block_kernel", __PRETTY_FUNCTION__, grid, kThreads);
  hipLaunchKernelGGL((quantize_e4m3_block_kernel<D, BF16, ROTATE>), dim3(grid), dim3(kThreads), 0, s, args);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <int D>
fa_status dispatch_quant(const QuantArgs& args, int grid, bool bf16, bool rotate, hipStream_t s) {
  if (bf16) return rotate ? launch_quant<D, true, true>(args, grid, s) : launch_quant<D, true, false>(args, grid, s);
  return rotate ? launch_quant<D, false, true>(args, grid, s) : launch_quant<D, false, false>(args, grid, s);
}

bool aligned(const void* p, size_t n) { return ((uintptr_t)p % n) == 0; }

}  // namespace

extern "C" {

fa_status fa_quantize_e4m3_block(const void* x, fa_dtype in_dtype, int B, int N, int Hx, int d,
                                 const float* signs, void* codes, unsigned char* scales,
                                 void* stream) {
  if (B < 1 || N < 1 || Hx < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (in_dtype != FA_DTYPE_F16 && in_dtype != FA_DTYPE_BF16) {
    return in_dtype == FA_DTYPE_FP8_E4M3 ? FA_ERR_UNSUPPORTED : FA_ERR_INVALID_ARG;
  }
  if ((long long)B * N * Hx * d >= (1LL << 31)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!x || !codes || !scales) return FA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, 8) || (signs && !aligned(signs, 16))) return FA_ERR_INVALID_ARG;
  QuantArgs args;
  args.x = x;
  args.signs = signs;
  args.codes = (uint8_t*)codes;
  args.scales = scales;
  args.N = N;
  args.Hx = Hx;
  args.nb = (N + kRows - 1) / kRows;
  const long long grid = (long long)B * Hx * args.nb;
  if (grid > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = in_dtype == FA_DTYPE_BF16;
  if (d == 128) return dispatch_quant<128>(args, (int)grid, bf16, signs != nullptr, s);
  return dispatch_quant<64>(args, (int)grid, bf16, signs != nullptr, s);
}

}  // extern "C"
