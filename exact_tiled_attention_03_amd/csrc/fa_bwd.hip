// fa_bwd.hip -- gradient of the exact attention forward for gfx950 (MI355X), and its C ABI.
//
// The pages report training speed-ups for the tiled method (abstracts of "FlashAttention:
// Fast and Memory-Efficient Exact Attention with IO-Awareness" and "FlashAttention-2:
// Faster Attention with Better Parallelism and Work Partitioning") but print no backward
// algorithm. This is the analytic gradient of the forward definition for an upstream dO,
// with no gradient through lse, computed the same I/O-aware way as the forward: the
// probabilities are recomputed tile by tile from Q, K and the saved lse, so no N x N
// matrix reaches HBM.
//     D_i   = <dO_i, O_i>                                   (preprocess kernel)
//     P_ij  = exp(scale <q_i, k_j> - lse_i)                 (masked pairs: 0)
//     dV_j  = sum_i P_ij dO_i,   dS_ij = P_ij (<dO_i, v_j> - D_i)
//     dK_j  = scale sum_i dS_ij q_i,   dQ_i = scale sum_j dS_ij k_j
// With grouped-query attention dK and dV of a key/value head sum over its query heads.
//
// gfx950 mapping (64-lane wavefronts):
//   * dK/dV kernel (v_mfma_f32_16x16x32): one workgroup of 8 wavefronts per (batch, K/V
//     head, 128 keys), each wavefront owning 16 keys, whose K and V rows stay in VGPRs as
//     MFMA B operands. It walks every query tile (64 rows) of every query head of the
//     group, last tile first: S = Q K^T and dP = dO V^T come out with one key per lane
//     (MFMA columns), so P and dS are lane-local elementwise work, and they leave the
//     accumulator already in the B-operand layout of dV^T += dO^T P and dK^T += Q^T dS
//     (queries consumed in a permuted order that the transposed Q^T / dO^T tiles in LDS
//     are written in). dK and dV accumulate in registers over all query tiles: no atomics,
//     deterministic. A tile runs as six software-pipelined phases (the S/dP MFMAs of its
//     four 16-query blocks, then the dV/dK MFMAs of its two 32-query chunks): each phase's
//     MFMAs cover the LDS reads of the next phase and the softmax of the block before, and
//     only tiles on the causal diagonal pay for the mask.
//   * dQ kernel (v_mfma_f32_32x32x16): one workgroup of 8 wavefronts per (batch, head, 256
//     queries), the forward's orientation: S^T = K Q^T and dP^T = V dO^T with one query
//     per lane, then dQ^T += K^T dS^T with K^T staged transposed in LDS. A 64-key tile
//     runs as phases over its two 32-key blocks, and only a ragged last tile or a causal
//     diagonal tile runs the masked body.
//   * Tiles are double-buffered in LDS with one barrier per tile. The global loads of the
//     next tile (dQ) or of the tile after it (dK/dV, two register sets) are in flight while
//     the current one is computed. Eight wavefronts share each LDS tile, two per SIMD, so
//     that one's MFMAs overlap the other's exponentials and LDS reads.
//   * Every swizzled LDS offset is one per-lane base XOR a constant plus an immediate; the
//     bases are formed per tile behind an empty asm, so the compiler neither holds every
//     offset in registers across the tile loop nor spills them.
//   * LDS bank conflicts were measured per access pattern with SQ_LDS_BANK_CONFLICT; every
//     tile read and staging write here is conflict-free. Writes behave as 32 banks x 4 B
//     served to 8 consecutive lanes (16-byte writes) or 16 consecutive lanes (8-byte
//     writes) at a time, so the transposed 8-byte writes need the 16 lanes of a group to
//     cover all 32 banks: each group holds two row groups whose slots fill the two halves
//     of a 16-byte chunk, times eight dims spread over the eight chunk positions.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "fa.h"
#include "fa_env.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;          // preprocess kernel
// dK/dV kernel: keys per wavefront and wavefronts per workgroup. The kernel is written for
// any multiple of 16 keys; 32 keys halve the LDS reads per MFMA but need one wavefront per
// SIMD for their registers, and measured 11% slower than two wavefronts of 16 keys.
// s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt not waited for. Both gradient kernels
// wait for all of their prologue loads before the tile loop. Without that wait the
// compiler's wait analysis merges the loop's entry state, in which the loads of the
// operands kept in registers may still be in flight, into the loop head, and then waits
// inside every tile for those loads and for every load issued after them, the next
// tile's staging loads included (3% of the gradient's time at B16 H16 N2048 d128).
constexpr int kVmcnt0 = 0x0F70;
constexpr int kKeysPerWaveKV = 16;
constexpr int kWavesKV = 128 / kKeysPerWaveKV;
constexpr int kWavesQ = 8;             // dQ kernel: wavefronts per workgroup, 32 queries each
constexpr float kLog2e = 1.4426950408889634f;

struct Bf16 {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float x, float y) {
    bf16x2 r = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(unsigned, r);
  }
  static __device__ __forceinline__ float lo(unsigned w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
};
struct F16 {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float x, float y) {
    f16x2 r = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(unsigned, r);
  }
  static __device__ __forceinline__ float lo(unsigned w) { return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu)); }
  static __device__ __forceinline__ float hi(unsigned w) { return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16)); }
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;          // workspace: D = rowsum(dO * O), [B][H][N]
  void* dq;
  void* dk;
  void* dv;
  int B, H, Hkv, N, group;
  float c;               // scale * log2(e)
  float scale;
  int tiles;             // workgroup tiles along the sequence for this kernel
  int total;             // workgroups in the grid
};

// Workgroup L runs on XCD L % 8; give each XCD one contiguous range of the logical list
// so that workgroups sharing inputs share an L2.
__device__ __forceinline__ int logical_index(int L, int total) {
  const int xcd = L & 7, slot = L >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

template <typename T>
__device__ __forceinline__ T lds_read(const unsigned char* base, int byte) {
  return *(const T*)(base + byte);
}

// LDS layouts of an R-row x D tile of 16-bit elements:
//   row-major (dQ kernel): 16-byte chunk c of row r at r*2D + ((c ^ rswz(r)) * 16), where
//     rswz(r) takes distinct values on rows r, r+1, r+2, r+3 and on r, r+4, r+8, r+12,
//     which keeps the 32-row reads of the 32x32x16 A operand conflict-free;
//   transposed: element (row x, dim t) at t*2R + 16 * ((slot/8) ^ (t/2) ^ ((t/16) % 4)) +
//     2 * (slot%8), with rows in slot order
//     slot(x) = 16(x/16) + 8((x%8)/4) + 4((x%16)/8) + x%4 (dQ kernel) or
//     slot32(x) (dK/dV kernel), the order in which an MFMA accumulator (rows
//     8(i/4) + 4(l/32) + i%4 of lane l) hands its rows to the next MFMA's k index. Reads
//     of 16 or 32 consecutive dims at one slot and the staging writes of dims 8c + e,
//     c = 0..7, both land on distinct banks.
__device__ __forceinline__ int rswz(int r) {
  const int x = r & 3;
  return ((x << 1) ^ (x << 2)) ^ ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int rm_byte(int r, int chunk) {
  return r * (2 * D) + (((chunk ^ rswz(r)) & (D / 8 - 1)) << 4);
}
template <int R>
__device__ __forceinline__ int tr_byte(int dim, int slot) {
  constexpr int kChunks = R / 8;
  return dim * (2 * R) + ((((slot >> 3) ^ (dim >> 1) ^ ((dim >> 4) & 3)) & (kChunks - 1)) << 4) + ((slot & 7) << 1);
}
__device__ __forceinline__ int slot_of(int x) {
  return (x & ~15) + (((x & 7) >> 2) << 3) + (((x & 15) >> 3) << 2) + (x & 3);
}

// Staging unit (row group g = rows 4g..4g+3, chunk c = dims 8c..8c+7) of lane sl of
// wavefront sw within a staging group of 16 * kChunks lanes. Lanes 8k..8k+7 take eight
// consecutive chunks of one row (a whole 128-byte line per load), lanes 8..15 of each 16
// the row group whose slots fill the other half of the same 16-byte chunks: bit kHalfBit
// of g is the slot function's half bit (bit 1 for slot(), bit 2 for slot32()).
template <int kChunks, int kHalfBit>
__device__ __forceinline__ void staging_unit(int sl, int sw, int& g, int& c) {
  static_assert(kChunks % 8 == 0 && (kHalfBit == 1 || kHalfBit == 2), "unit mapping");
  constexpr int kWavesPerRow = kChunks / 8;
  c = (sl & 7) + 8 * (sw % kWavesPerRow);
  const int h = (sl >> 3) & 1, q = sl >> 4;
  const int low = kHalfBit == 2 ? (q | (h << 2)) : ((q & 1) | (h << 1) | ((q >> 1) << 2));
  g = low | ((sw / kWavesPerRow) << 3);
}

// Per-lane bases of the staging writes of unit (g, c): since rswz(4g + j) =
// rswz(j) ^ (g % 4) and the transposed swizzle of dim 8c + e is that of 8c XOR e/2, every
// write is one base XOR a constant plus an immediate:
//   rm_byte(4g + j, c)      = (rm_stage_base ^ 16 rswz(j)) + 2D j
//   tr_byte(8c + e, slot_of(4g)) = (tr_stage_base ^ 16 (e/2)) + 2R e
template <int D>
__device__ __forceinline__ int rm_stage_base(int g, int c) {
  return 4 * g * (2 * D) + (((c ^ (g & 3)) & (D / 8 - 1)) << 4);
}
template <int R>
__device__ __forceinline__ int tr_stage_base(int g, int c) {
  const int s0 = slot_of(4 * g);
  return 8 * c * (2 * R) + ((((s0 >> 3) ^ (4 * (c & 1)) ^ ((c >> 1) & 3)) & (R / 8 - 1)) << 4) + ((s0 & 7) << 1);
}

// Stage loaded rows (4 consecutive rows x 8 dims per unit) into LDS, row-major and/or
// transposed, from the unit's write bases. rows[j] holds dims 8c..8c+7 of row 4g + j.
template <int D, int R, bool ROWMAJOR, bool TRANSPOSED>
__device__ __forceinline__ void stage_rows(unsigned char* rm, unsigned char* tr, int rmw, int trw, const u32x4 (&rows)[4]) {
  if constexpr (ROWMAJOR) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u32x4*)(rm + ((rmw ^ ((rswz(j) & (D / 8 - 1)) << 4)) + j * (2 * D))) = rows[j];
  }
  if constexpr (TRANSPOSED) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x2 w;
      w[0] = __builtin_amdgcn_perm(rows[1][e >> 1], rows[0][e >> 1], sel);
      w[1] = __builtin_amdgcn_perm(rows[3][e >> 1], rows[2][e >> 1], sel);
      *(u32x2*)(tr + ((trw ^ ((e >> 1) << 4)) + e * (2 * R))) = w;
    }
  }
}

// ---- preprocess: D_i = <dO_i, O_i> in float32 ----------------------------------------
template <typename Ops, int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(BwdArgs a) {
  constexpr int kLanes = D / 8;                    // lanes per row, 8 elements each
  const int row = blockIdx.x * (kThreads / kLanes) + threadIdx.x / kLanes;   // (b, i, h) flattened
  const int c = threadIdx.x % kLanes;
  const int rows = a.B * a.N * a.H;
  float s = 0.0f;
  if (row < rows) {
    const u32x4 x = *(const u32x4*)((const uint16_t*)a.o + (size_t)row * D + c * 8);
    const u32x4 y = *(const u32x4*)((const uint16_t*)a.dout + (size_t)row * D + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) s += Ops::lo(x[w]) * Ops::lo(y[w]) + Ops::hi(x[w]) * Ops::hi(y[w]);
  }
#pragma unroll
  for (int m = 1; m < kLanes; m <<= 1) s += __shfl_xor(s, m, 64);
  if (row < rows && c == 0) {
    const int h = row % a.H, i = (row / a.H) % a.N, b = row / (a.H * a.N);
    a.delta[((size_t)b * a.H + h) * a.N + i] = s;
  }
}

// ---- dK / dV -------------------------------------------------------------------------
// v_mfma_f32_16x16x32 layouts (lane l, g = l/16, c = l%16): A[m = c][k = 8g + i],
// B[k = 8g + i][n = c], C[row = 4g + i][col = c]. Two 16-row accumulator blocks hand
// their 32 rows to the next MFMA's k index in the order
//   slot(x) = 32(x/32) + 8((x%16)/4) + 4((x%32)/16) + x%4,
// in which the transposed Q^T / dO^T tiles are written.
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <typename Ops>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma16<Bf16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16<F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ int slot32_of(int x) {
  return (x & ~31) + (((x & 15) >> 2) << 3) + (((x & 31) >> 4) << 2) + (x & 3);
}
template <int D>
__device__ __forceinline__ int rm16_byte(int r, int chunk) {       // row-major, 16-byte chunks
  return r * (2 * D) + ((chunk ^ (r & (D / 8 - 1))) << 4);
}

template <typename Ops, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kWavesKV) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int kKb = kKeysPerWaveKV / 16;   // 16-key blocks per wavefront
  constexpr int kBk = kKeysPerWaveKV * kWavesKV;   // keys per workgroup
  constexpr int kBq = 64;                  // queries per tile
  constexpr int kKsteps = D / 32;          // k-steps of the 16x16x32 MFMA over d
  constexpr int kDblocks = D / 16;         // 16-dim blocks of dK^T / dV^T
  constexpr int kTile = kBq * D * 2;       // one 16-bit tile
  constexpr int kBuf = 4 * kTile + 2 * kBq * 4;   // Q, dO (row-major), Q^T, dO^T, lse2, D
  constexpr int kChunks = D / 8;
  constexpr int kUnits = (kBq / 4) * kChunks;      // staging units (4 rows x 8 dims) per tensor
  // either every thread stages one unit of Q and one of dO, or the first kUnits threads
  // stage Q and the next kUnits dO
  constexpr bool kBoth = kUnits == 64 * kWavesKV;
  constexpr int kUpt = kBoth ? 2 : 1;
  static_assert(kUnits % 64 == 0 && (kBoth || 2 * kUnits <= 64 * kWavesKV), "staging units fill whole wavefronts");
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kBuf];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int lg = logical_index(blockIdx.x, a.total);
  const int kt = lg % a.tiles;
  const int bh = lg / a.tiles;               // b * Hkv + hk
  const int hk = bh % a.Hkv, b = bh / a.Hkv;
  const int N = a.N;
  const int k0 = kt * kBk;
  const int kw0 = k0 + kKeysPerWaveKV * wave;  // this wavefront's first key
  // this lane's keys (MFMA columns): kw0 + 16kb + c
  const size_t q_stride = (size_t)a.H * D, kv_stride = (size_t)a.Hkv * D;

  // K and V rows of the lane's keys as B operands: dims 32ks + 8g .. +7
  u32x4 kreg[kKb][kKsteps], vreg[kKb][kKsteps];
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb) {
    const int kr = min(kw0 + 16 * kb + c, N - 1);
    const uint16_t* kp = (const uint16_t*)a.k + ((size_t)b * N + kr) * kv_stride + (size_t)hk * D + g * 8;
    const uint16_t* vp = (const uint16_t*)a.v + ((size_t)b * N + kr) * kv_stride + (size_t)hk * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < kKsteps; ++ks) {
      kreg[kb][ks] = *(const u32x4*)(kp + ks * 32);
      vreg[kb][ks] = *(const u32x4*)(vp + ks * 32);
    }
  }
  f32x4 dkT[kKb][kDblocks], dvT[kKb][kDblocks];   // C[dim][key]
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
    for (int i = 0; i < kDblocks; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dkT[kb][i][e] = dvT[kb][i][e] = 0.0f;

  const int qt0 = CAUSAL ? k0 / kBq : 0;
  const int nqt = (N + kBq - 1) / kBq;
  const int per_head = nqt - qt0;
  const int T = per_head * a.group;

  // staging unit = rows 4sg..4sg+3, dims 8sc..8sc+7 of Q (which 0) or dO (which 1)
  const int su = kBoth ? tid : tid % kUnits, which = kBoth ? 0 : tid / kUnits;   // which 2+: none
  int sg, sc;
  staging_unit<kChunks, 2>(su & 63, su >> 6, sg, sc);
  // two register sets of staged rows: the loads of tile t+2 go out when tile t starts, a
  // whole tile before its rows are needed in LDS (the Q/dO tiles come from L2 or HBM, and
  // one tile of lead left the staging waiting on them)
  u32x4 rows[2][kUpt][4];
  float lse_st[2] = {0.0f, 0.0f};
  // query tiles from the last one down, the heads of the group interleaved (head fastest),
  // so that the workgroups of one K/V head read the same Q/dO tile of the same head at
  // about the same time and share it in L2: under the causal mask they stop at different
  // tiles, and a head-major walk put them on different heads' rows (16 MiB per K/V head
  // at N = 8192, four times an XCD's L2)
  auto tile_coords = [&](int t, int& h, int& q0) __attribute__((always_inline)) {
    h = hk * a.group + t % a.group;
    q0 = (nqt - 1 - t / a.group) * kBq;
  };
  auto load_tile = [&](int t, auto set_c) __attribute__((always_inline)) {
    constexpr int st = decltype(set_c)::value;
    int h, q0;
    tile_coords(t, h, q0);
#pragma unroll
    for (int u = 0; u < kUpt; ++u) {
      const int wh = kBoth ? u : which;
      if (wh < 2) {
        const uint16_t* src = (const uint16_t*)(wh == 0 ? a.q : a.dout);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = min(q0 + 4 * sg + j, N - 1);
          rows[st][u][j] = *(const u32x4*)(src + ((size_t)b * N + r) * q_stride + (size_t)h * D + sc * 8);
        }
      }
    }
    if (tid < 2 * kBq) {                     // lse (scaled to base 2) then D
      const int r = q0 + (tid % kBq);
      const size_t off = ((size_t)b * a.H + h) * N + min(r, N - 1);
      if (tid < kBq) lse_st[st] = r < N ? a.lse[off] * kLog2e : INFINITY;     // rows past the end: P = 0
      else lse_st[st] = r < N ? a.delta[off] : 0.0f;
    }
  };
  // staging-write bases: rm16_byte(4sg + j, sc) = (rm_w0 ^ 16j) + 2D j and
  // tr_byte(8sc + e, slot32(4sg)) = (tr_w0 ^ 16(e/2)) + 2 kBq e
  const int rm_w0 = 4 * sg * (2 * D) + (((sc ^ (4 * (sg & 3))) & (kChunks - 1)) << 4);
  const int tr_w0 = [&] {
    const int s0 = slot32_of(4 * sg);
    return 8 * sc * (2 * kBq) + ((((s0 >> 3) ^ (4 * (sc & 1)) ^ ((sc >> 1) & 3)) & 7) << 4) + ((s0 & 7) << 1);
  }();
  // tile rows of register set st into LDS buffer st (a tile's buffer and set are both its
  // parity)
  auto store_tile = [&](auto set_c) __attribute__((always_inline)) {
    constexpr int st = decltype(set_c)::value, buf = st;
    // opaque per call: the write offsets are formed here, not held across the loop
    int rmw = buf * kBuf + rm_w0, trw = buf * kBuf + tr_w0;
    asm volatile("" : "+v"(rmw), "+v"(trw));
#pragma unroll
    for (int u = 0; u < kUpt; ++u) {
      const int wh = kBoth ? u : which;
      if (wh < 2) {
        unsigned char* rm = lds + wh * kTile;
        unsigned char* tr = lds + (2 + wh) * kTile;
#pragma unroll
        for (int j = 0; j < 4; ++j) *(u32x4*)(rm + ((rmw ^ (j << 4)) + j * (2 * D))) = rows[st][u][j];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
          u32x2 w;
          w[0] = __builtin_amdgcn_perm(rows[st][u][1][e >> 1], rows[st][u][0][e >> 1], sel);
          w[1] = __builtin_amdgcn_perm(rows[st][u][3][e >> 1], rows[st][u][2][e >> 1], sel);
          *(u32x2*)(tr + ((trw ^ ((e >> 1) << 4)) + e * (2 * kBq))) = w;
        }
      }
    }
    unsigned char* base = lds + buf * kBuf;
    if (tid < 2 * kBq) ((float*)(base + 4 * kTile))[tid] = lse_st[st];
  };

  // Each 64-query tile runs as six phases whose MFMAs hide the next phase's LDS reads
  // and the previous phase's softmax arithmetic (the other wavefront of the SIMD covers
  // only what these leave exposed): S(c,h) are the S/dP MFMAs of 16-query block h of
  // 32-query chunk c, E(c,h) its probabilities and dS, V(c) the dV/dK MFMAs of chunk c:
  //   S(0,0) | S(0,1) E(0,0) | S(1,0) E(0,1) | S(1,1) E(1,0) | V(0) E(1,1) | V(1) staging
  // Read bases (a tile's buffer offset plus these, formed per tile): the swizzles are XORs
  // on bits that the block offsets leave clear, so
  //   rm16_byte(32qc + 16half + c, 4ks + g)  = (s_lane ^ 64ks) + 2D (32qc + 16half)
  //   tr_byte(16dbk + c, 32qc + 8g)          = (v_lane ^ 16(4qc ^ dbk%4)) + 2 kBq 16dbk
  const int s_lane = c * (2 * D) + (((g ^ c) & (kChunks - 1)) << 4);
  const int v_lane = c * (2 * kBq) + (((g ^ (c >> 1)) & 7) << 4);
  auto s_read = [&](int sb, int qc, int half, u32x4 (&qa)[kKsteps], u32x4 (&da)[kKsteps])
      __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < kKsteps; ++ks) {
      const int off = (sb ^ (ks << 6)) + (qc * 32 + half * 16) * (2 * D);
      qa[ks] = lds_read<u32x4>(lds, off);
      da[ks] = lds_read<u32x4>(lds + kTile, off);
    }
  };
  auto s_mfma = [&](const u32x4 (&qa)[kKsteps], const u32x4 (&da)[kKsteps], f32x4 (&sacc)[kKb], f32x4 (&dpacc)[kKb])
      __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc[kb][e] = dpacc[kb][e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kKsteps; ++ks)
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb) {
        sacc[kb] = mfma16<Ops>(qa[ks], kreg[kb][ks], sacc[kb]);
        dpacc[kb] = mfma16<Ops>(da[ks], vreg[kb][ks], dpacc[kb]);
      }
  };
  // P and dS of one 16-query block into k-slots 8g + 4*half + i of the chunk's B operands.
  // Only the causal mask is applied: P and dS of a key past the end reach nothing but that
  // key's own dK / dV rows, which are never stored, and query rows past the end have
  // lse = +inf, so P = dS = 0 there.
  // lse (base 2) and D of the lane's four query rows of a 16-query block
  auto stats_read = [&](const unsigned char* base, int qc, int half, float4& l4, float4& d4) __attribute__((always_inline)) {
    const float* lse2 = (const float*)(base + 4 * kTile);
    const int q4 = qc * 32 + half * 16 + 4 * g;
    l4 = *(const float4*)(lse2 + q4);
    d4 = *(const float4*)(lse2 + kBq + q4);
  };
  auto softmax = [&](auto masked_c, int q0, int qc, int half, const float4& l4, const float4& d4,
                     const f32x4 (&sacc)[kKb], const f32x4 (&dpacc)[kKb], u32x4 (&pb)[kKb], u32x4 (&db)[kKb])
      __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked_c)::value;
    // accumulator i: query row qc*32 + half*16 + 4g + i, key column c of block kb
    const int q4 = qc * 32 + half * 16 + 4 * g;
    const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
    const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) {
      const int past = kw0 + 16 * kb + c - (q0 + q4);   // key - query of accumulator 0
      float pv[4], dsv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], a.c, -lv[i]));
        if (kMasked && past > i) p = 0.0f;
        pv[i] = p;
        dsv[i] = p * (dpacc[kb][i] - dv4[i]);
      }
      pb[kb][2 * half] = Ops::pack2(pv[0], pv[1]);
      pb[kb][2 * half + 1] = Ops::pack2(pv[2], pv[3]);
      db[kb][2 * half] = Ops::pack2(dsv[0], dsv[1]);
      db[kb][2 * half + 1] = Ops::pack2(dsv[2], dsv[3]);
    }
  };
  // A operands of dV^T += dO^T P and dK^T += Q^T dS: dim 16 dbk + c, slots qc*32 + 8g .. +7
  auto v_read = [&](int vb, int qc, int lo, int hi, u32x4 (&da)[kDblocks], u32x4 (&qa)[kDblocks])
      __attribute__((always_inline)) {
#pragma unroll
    for (int dbk = lo; dbk < hi; ++dbk) {
      const int off = (vb ^ ((4 * qc ^ (dbk & 3)) << 4)) + dbk * 16 * (2 * kBq);
      da[dbk] = lds_read<u32x4>(lds + 3 * kTile, off);
      qa[dbk] = lds_read<u32x4>(lds + 2 * kTile, off);
    }
  };
  auto v_mfma = [&](const u32x4 (&da)[kDblocks], const u32x4 (&qa)[kDblocks], const u32x4 (&pb)[kKb], const u32x4 (&db)[kKb])
      __attribute__((always_inline)) {
#pragma unroll
    for (int dbk = 0; dbk < kDblocks; ++dbk)
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb) {
        dvT[kb][dbk] = mfma16<Ops>(da[dbk], pb[kb], dvT[kb][dbk]);
        dkT[kb][dbk] = mfma16<Ops>(qa[dbk], db[kb], dkT[kb][dbk]);
      }
  };
  constexpr int kSM = 2 * kKsteps * kKb;     // MFMAs of an S phase
  constexpr int kVM = 2 * kDblocks * kKb;    // MFMAs of a V phase

  load_tile(0, std::integral_constant<int, 0>{});
  store_tile(std::integral_constant<int, 0>{});
  if (1 < T) load_tile(1, std::integral_constant<int, 1>{});
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();

  // tile t of parity par: loads of tile t+2 into register set par (stored at the end of
  // tile t-1), reads from buffer par, tile t+1 staged from set par^1 into buffer par^1
  auto tile_iter = [&](int t, auto par_c) __attribute__((always_inline)) {
    constexpr int par = decltype(par_c)::value;
    if (t + 2 < T) load_tile(t + 2, std::integral_constant<int, par>{});
    int h, q0;
    tile_coords(t, h, q0);
    (void)h;
    const unsigned char* base = lds + par * kBuf;
    int sb = par * kBuf + s_lane, vb = par * kBuf + v_lane;
    asm volatile("" : "+v"(sb), "+v"(vb));
    auto tile_body = [&](auto masked_c) __attribute__((always_inline)) {
      u32x4 sq0[kKsteps], sd0[kKsteps], sq1[kKsteps], sd1[kKsteps];
      u32x4 va0[kDblocks], vb0[kDblocks], va1[kDblocks], vb1[kDblocks];
      f32x4 sa0[kKb], sp0[kKb], sa1[kKb], sp1[kKb];
      u32x4 pb0[kKb], db0[kKb], pb1[kKb], db1[kKb];
      float4 l0, d0, l1, d1;                 // statistics of the next two softmax blocks
      constexpr int kHalfD = kDblocks / 2;
      // S(0,0), then E(0,0)'s statistics and S(0,1)'s reads in its second half
      s_read(sb, 0, 0, sq0, sd0);
      s_mfma(sq0, sd0, sa0, sp0);
      stats_read(base, 0, 0, l0, d0);
      s_read(sb, 0, 1, sq1, sd1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kKsteps, 0);
#pragma unroll
      for (int i = 0; i < kSM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i == kSM / 2 - 1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        if (i >= kSM / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2 * kKsteps / (kSM / 2), 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // S(0,1) | E(0,0) | E(0,1)'s statistics, reads of S(1,0)
      s_mfma(sq1, sd1, sa1, sp1);
      softmax(masked_c, q0, 0, 0, l0, d0, sa0, sp0, pb0, db0);
      stats_read(base, 0, 1, l1, d1);
      s_read(sb, 1, 0, sq0, sd0);
#pragma unroll
      for (int i = 0; i < kSM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i == kSM / 2 - 1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        if (i >= kSM / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2 * kKsteps / (kSM / 2), 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // S(1,0) | E(0,1) | E(1,0)'s statistics, reads of S(1,1)
      s_mfma(sq0, sd0, sa0, sp0);
      softmax(masked_c, q0, 0, 1, l1, d1, sa1, sp1, pb0, db0);
      stats_read(base, 1, 0, l0, d0);
      s_read(sb, 1, 1, sq1, sd1);
#pragma unroll
      for (int i = 0; i < kSM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i == kSM / 2 - 1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        if (i >= kSM / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2 * kKsteps / (kSM / 2), 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // S(1,1) | E(1,0) | E(1,1)'s statistics, reads of the first half of V(0)
      s_mfma(sq1, sd1, sa1, sp1);
      softmax(masked_c, q0, 1, 0, l0, d0, sa0, sp0, pb1, db1);
      stats_read(base, 1, 1, l1, d1);
      v_read(vb, 0, 0, kHalfD, va0, vb0);
#pragma unroll
      for (int i = 0; i < kSM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i == kSM / 2 - 1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        if (i >= kSM / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2 * kHalfD / (kSM / 2), 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // V(0) | E(1,1) | the second half of V(0)'s reads, then the first half of V(1)'s
      v_read(vb, 0, kHalfD, kDblocks, va0, vb0);
      v_mfma(va0, vb0, pb0, db0);
      softmax(masked_c, q0, 1, 1, l1, d1, sa1, sp1, pb1, db1);
      v_read(vb, 1, 0, kHalfD, va1, vb1);
#pragma unroll
      for (int i = 0; i < kVM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 2 * kHalfD || i >= kVM / 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // V(1) | the second half of its reads | staging of the next tile
      v_read(vb, 1, kHalfD, kDblocks, va1, vb1);
      v_mfma(va1, vb1, pb1, db1);
      store_tile(std::integral_constant<int, par ^ 1>{});   // after the last tile: an unused buffer
#pragma unroll
      for (int i = 0; i < kVM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 2 * kHalfD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    if (!CAUSAL || kw0 + kKeysPerWaveKV - 1 <= q0) {
      tile_body(std::false_type{});          // every key at or before every query of the tile
    } else if (kw0 <= q0 + kBq - 1) {
      tile_body(std::true_type{});
    } else {
      store_tile(std::integral_constant<int, par ^ 1>{});               // all queries precede the keys: nothing to add
    }
    __syncthreads();
  };
  for (int t = 0; t < T; t += 2) {
    tile_iter(t, std::integral_constant<int, 0>{});
    if (t + 1 < T) tile_iter(t + 1, std::integral_constant<int, 1>{});
  }

  // epilogue: lane holds dims 16dbk + 4g + 0..3 of its keys
#pragma unroll
  for (int kb = 0; kb < kKb; ++kb) {
    const int key = kw0 + 16 * kb + c;
    if (key < N) {
      const size_t off = ((size_t)b * N + key) * kv_stride + (size_t)hk * D;
#pragma unroll
      for (int dbk = 0; dbk < kDblocks; ++dbk) {
        const int dim = dbk * 16 + 4 * g;
        u32x2 wk, wv;
        wk[0] = Ops::pack2(dkT[kb][dbk][0] * a.scale, dkT[kb][dbk][1] * a.scale);
        wk[1] = Ops::pack2(dkT[kb][dbk][2] * a.scale, dkT[kb][dbk][3] * a.scale);
        wv[0] = Ops::pack2(dvT[kb][dbk][0], dvT[kb][dbk][1]);
        wv[1] = Ops::pack2(dvT[kb][dbk][2], dvT[kb][dbk][3]);
        *(u32x2*)((uint16_t*)a.dk + off + dim) = wk;
        *(u32x2*)((uint16_t*)a.dv + off + dim) = wv;
      }
    }
  }
}

// ---- dQ ------------------------------------------------------------------------------
template <typename Ops, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kWavesQ) void bwd_dq_kernel(BwdArgs a) {
  constexpr int kBq = 32 * kWavesQ;        // queries per workgroup, 32 per wavefront
  constexpr int kBk = 64;                  // keys per tile
  constexpr int kKb = kBk / 32;            // 32-key blocks per tile
  constexpr int kKsteps = D / 16;
  constexpr int kDblocks = D / 32;
  constexpr int kTile = kBk * D * 2;
  constexpr int kBuf = 3 * kTile;          // K, V (row-major), K^T
  constexpr int kChunks = D / 8;
  constexpr int kUnits = (kBk / 4) * kChunks;
  static_assert(kUnits % 64 == 0 && kUnits <= 64 * kWavesQ, "staging units fill whole wavefronts");
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kBuf];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int lg = logical_index(blockIdx.x, a.total);
  // logical order (b, hk, query tile, head in group): heads sharing K/V are neighbours
  const int gm = lg % a.group;
  int t_ = lg / a.group;
  int qt = t_ % a.tiles;
  t_ /= a.tiles;
  const int hk = t_ % a.Hkv, b = t_ / a.Hkv;
  if (CAUSAL) qt = a.tiles - 1 - qt;       // longest first
  const int h = hk * a.group + gm;
  const int N = a.N;
  const int q0 = qt * kBq;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + l32;
  const size_t q_stride = (size_t)a.H * D, kv_stride = (size_t)a.Hkv * D;

  u32x4 qreg[kKsteps], dreg[kKsteps];
  {
    const int r = min(qi, N - 1);
    const size_t off = ((size_t)b * N + r) * q_stride + (size_t)h * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < kKsteps; ++ks) {
      qreg[ks] = *(const u32x4*)((const uint16_t*)a.q + off + ks * 16);
      dreg[ks] = *(const u32x4*)((const uint16_t*)a.dout + off + ks * 16);
    }
  }
  const size_t lrow = ((size_t)b * a.H + h) * N + min(qi, N - 1);
  const float lse2 = qi < N ? a.lse[lrow] * kLog2e : INFINITY;
  const float dlt = qi < N ? a.delta[lrow] : 0.0f;
  f32x16 dqT[kDblocks];                      // C[dim][query]
#pragma unroll
  for (int i = 0; i < kDblocks; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqT[i][e] = 0.0f;

  const int kv_end = CAUSAL ? min(N, q0 + kBq) : N;
  const int T = (kv_end + kBk - 1) / kBk;

  const bool stager = tid < kUnits;
  int sg, sc;
  staging_unit<kChunks, 1>(lane, wave, sg, sc);
  u32x4 krows[4], vrows[4];
  auto load_tile = [&](int t) __attribute__((always_inline)) {
    if (stager) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = min(t * kBk + 4 * sg + j, N - 1);
        const size_t off = ((size_t)b * N + r) * kv_stride + (size_t)hk * D + sc * 8;
        krows[j] = *(const u32x4*)((const uint16_t*)a.k + off);
        vrows[j] = *(const u32x4*)((const uint16_t*)a.v + off);
      }
    }
  };
  const int rmw0 = rm_stage_base<D>(sg, sc), trw0 = tr_stage_base<kBk>(sg, sc);
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
    unsigned char* base = lds + buf * kBuf;
    if (stager) {
      // opaque copies: the write offsets are formed per call, not held across the loop
      int rmw = rmw0, trw = trw0;
      asm volatile("" : "+v"(rmw), "+v"(trw));
      stage_rows<D, kBk, true, true>(base, base + 2 * kTile, rmw, trw, krows);
      stage_rows<D, kBk, true, false>(base + kTile, nullptr, rmw, trw, vrows);
    }
  };

  // LDS read offsets. The swizzles are XORs on bits that the buffer and block offsets leave
  // clear, so every read is one per-lane base XOR a constant, plus an immediate:
  //   rm_byte(32kb + l32, 2ks + hi)            = (rm_lane ^ 32ks) + 32kb * 2D
  //   tr_byte(32dbk + l32, 32kb + 16t2 + 8hi) = (tr_lane ^ 16(4kb ^ 2(t2 ^ dbk%2))) + 4096dbk
  const int rm_lane = l32 * (2 * D) + (((hi ^ rswz(l32)) & (kChunks - 1)) << 4);
  const int tr_lane = l32 * (2 * kBk) + (((hi ^ ((l32 >> 1) & 7) ^ (l32 >> 4)) & 7) << 4);
  // S^T and dP^T of a 32-key block, then P and dS^T of it as B operands of dQ^T += K^T dS^T.
  // In both MFMA loops below the operand reads run ahead of their MFMAs (four reads for
  // S/dP, three for dQ) in the source order, and a scheduling barrier after each MFMA
  // keeps that order: left to itself, the scheduler put each read right before its MFMA
  // behind a full LDS wait (the dQ kernel 4-6% slower).
  auto s_mfma = [&](int rmb, int kb, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.0f;
    auto off = [&](int ks) { return (rmb ^ (ks << 5)) + kb * 32 * (2 * D); };
    u32x4 ka[kKsteps], va[kKsteps];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      ka[ks] = lds_read<u32x4>(lds, off(ks));
      va[ks] = lds_read<u32x4>(lds + kTile, off(ks));
    }
#pragma unroll
    for (int ks = 0; ks < kKsteps; ++ks) {
      if (ks + 2 < kKsteps) {
        ka[ks + 2] = lds_read<u32x4>(lds, off(ks + 2));
        va[ks + 2] = lds_read<u32x4>(lds + kTile, off(ks + 2));
      }
      s = Ops::mfma(ka[ks], qreg[ks], s);
      dp = Ops::mfma(va[ks], dreg[ks], dp);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Masks apply only where a key is past the end or (causal) after the lane's query.
  const int key_last = CAUSAL ? min(qi, N - 1) : N - 1;
  auto softmax = [&](auto masked_c, int j0, int kb, const f32x16& s, const f32x16& dp, u32x4 (&db)[2])
      __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked_c)::value;
    // accumulator e holds key j0 + 32kb + 4hi + 8(e/4) + e%4, visible up to key_last
    const int thr = key_last - (j0 + kb * 32 + 4 * hi);
    float dsv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], a.c, -lse2));
      if (kMasked && 8 * (e >> 2) + (e & 3) > thr) p = 0.0f;
      dsv[e] = p * (dp[e] - dlt);
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int w = 0; w < 4; ++w) db[t2][w] = Ops::pack2(dsv[8 * t2 + 2 * w], dsv[8 * t2 + 2 * w + 1]);
  };
  // dQ^T += K^T dS^T: A = K^T (dim 32 dbk + l32, slots kb*32 + 16 t2 + 8 hi .. +7)
  auto q_mfma = [&](int trb, int kb, const u32x4 (&db)[2]) __attribute__((always_inline)) {
    constexpr int kN = 2 * kDblocks;
    auto off = [&](int i) {
      const int t2 = i / kDblocks, dbk = i % kDblocks;
      return (trb ^ ((4 * kb ^ 2 * (t2 ^ (dbk & 1))) << 4)) + dbk * 32 * (2 * kBk);
    };
    u32x4 ka[kN];
#pragma unroll
    for (int i = 0; i < 3; ++i) ka[i] = lds_read<u32x4>(lds + 2 * kTile, off(i));
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      if (i + 3 < kN) ka[i + 3] = lds_read<u32x4>(lds + 2 * kTile, off(i + 3));
      dqT[i % kDblocks] = Ops::mfma(ka[i], db[i / kDblocks], dqT[i % kDblocks]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  load_tile(0);
  store_tile(0);
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();

  // S(0) E(0) | S(1) | dQ(0) E(1) | dQ(1) staging, two 32-key blocks per tile (the first
  // softmax overlaps the other wavefront of the SIMD: overlapping it with S(1) would hold
  // both blocks' accumulators)
  auto tile_body = [&](int t, auto masked_c) __attribute__((always_inline)) {
    if (t + 1 < T) load_tile(t + 1);
    // the tile's per-lane read bases, opaque to the compiler so that the offsets derived
    // from them are formed per tile rather than held in registers across the loop
    int rmb = (t & 1) * kBuf + rm_lane, trb = (t & 1) * kBuf + tr_lane;
    asm volatile("" : "+v"(rmb), "+v"(trb));
    const int j0 = t * kBk;
    f32x16 s0, dp0, s1, dp1;
    u32x4 db0[2], db1[2];
    s_mfma(rmb, 0, s0, dp0);
    __builtin_amdgcn_sched_barrier(0);
    softmax(masked_c, j0, 0, s0, dp0, db0);
    __builtin_amdgcn_sched_barrier(0);
    s_mfma(rmb, 1, s1, dp1);
    __builtin_amdgcn_sched_barrier(0);
    q_mfma(trb, 0, db0);
    softmax(masked_c, j0, 1, s1, dp1, db1);
    __builtin_amdgcn_sched_barrier(0);
    q_mfma(trb, 1, db1);
    store_tile((t + 1) & 1);   // after the last tile: an unused buffer
    __builtin_amdgcn_sched_barrier(0);
  };
  if (!CAUSAL) {
    // every tile but a ragged last one has all of its keys in range
    const int T_full = N / kBk;
    for (int t = 0; t < T_full; ++t) {
      tile_body(t, std::false_type{});
      __syncthreads();
    }
    for (int t = T_full; t < T; ++t) {
      tile_body(t, std::true_type{});
      __syncthreads();
    }
  } else {
    for (int t = 0; t < T; ++t) {
      const int j0 = t * kBk;
      if (j0 + kBk <= N && j0 + kBk - 1 <= qw0) {      // no key masked
        tile_body(t, std::false_type{});
      } else if (j0 <= qw0 + 31) {                    // some key at or before a query
        tile_body(t, std::true_type{});
      } else {
        if (t + 1 < T) load_tile(t + 1);
        store_tile((t + 1) & 1);
      }
      __syncthreads();
    }
  }

  if (qi < N) {
    const size_t off = ((size_t)b * N + qi) * q_stride + (size_t)h * D;
#pragma unroll
    for (int dbk = 0; dbk < kDblocks; ++dbk)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = dbk * 32 + 8 * g + 4 * hi;
        u32x2 w;
        w[0] = Ops::pack2(dqT[dbk][4 * g] * a.scale, dqT[dbk][4 * g + 1] * a.scale);
        w[1] = Ops::pack2(dqT[dbk][4 * g + 2] * a.scale, dqT[dbk][4 * g + 3] * a.scale);
        *(u32x2*)((uint16_t*)a.dq + off + dim) = w;
      }
  }
}

// ---- host ----------------------------------------------------------------------------
bool aligned(const void* p, size_t n) { return ((uintptr_t)p % n) == 0; }

template <typename Ops, int D, bool CAUSAL>
fa_status launch_bwd(BwdArgs args, hipStream_t s) {
  const int rows = args.B * args.N * args.H;
  const int per_block = kThreads / (D / 8);
  fa_env::log_launch("bwd_delta_kernel", __PRETTY_FUNCTION__, (rows + per_block - 1) / per_block, kThreads);
  hipLaunchKernelGGL((bwd_delta_kernel<Ops, D>), dim3((rows + per_block - 1) / per_block), dim3(kThreads), 0, s, args);
  if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
  BwdArgs kv = args;
  kv.tiles = (args.N + kKeysPerWaveKV * kWavesKV - 1) / (kKeysPerWaveKV * kWavesKV);
  kv.total = kv.tiles * args.Hkv * args.B;
  fa_env::log_launch("bwd_dkdv_kernel", __PRETTY_FUNCTION__, kv.total, 64 * kWavesKV);
  hipLaunchKernelGGL((bwd_dkdv_kernel<Ops, D, CAUSAL>), dim3(kv.total), dim3(64 * kWavesKV), 0, s, kv);
  if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
  BwdArgs qa = args;
  qa.tiles = (args.N + 32 * kWavesQ - 1) / (32 * kWavesQ);
  qa.total = qa.tiles * args.H * args.B;
  fa_env::log_launch("bwd_dq_kernel", __PRETTY_FUNCTION__, qa.total, 64 * kWavesQ);
  hipLaunchKernelGGL((bwd_dq_kernel<Ops, D, CAUSAL>), dim3(qa.total), dim3(64 * kWavesQ), 0, s, qa);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <typename Ops>
fa_status dispatch_bwd(const BwdArgs& args, int d, int causal, hipStream_t s) {
  if (d == 128) return causal ? launch_bwd<Ops, 128, true>(args, s) : launch_bwd<Ops, 128, false>(args, s);
  return causal ? launch_bwd<Ops, 64, true>(args, s) : launch_bwd<Ops, 64, false>(args, s);
}

fa_status check_bwd(int B, int H, int Hkv, int N, int d, int causal, fa_dtype dtype) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (Hkv > H || H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) {
    return dtype == FA_DTYPE_FP8_E4M3 ? FA_ERR_UNSUPPORTED : FA_ERR_INVALID_ARG;
  }
  if ((long long)B * N * H * d >= (1LL << 31)) return FA_ERR_INVALID_ARG;
  if ((long long)(N + 31) / 32 * H * B > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  return (size_t)B * H * N * sizeof(float);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                 int causal, float scale, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  fa_status st = check_bwd(B, H, Hkv, N, d, causal, dtype);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_INVALID_ARG;
  const void* p16[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : p16)
    if (!aligned(p, 16)) return FA_ERR_INVALID_ARG;
  if (!aligned(lse, 4) || !aligned(workspace, 4)) return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa_bwd_workspace_bytes(B, H, N)) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  BwdArgs args;
  args.q = q;
  args.k = k;
  args.v = v;
  args.o = o;
  args.dout = dout;
  args.lse = lse;
  args.delta = (float*)workspace;
  args.dq = dq;
  args.dk = dk;
  args.dv = dv;
  args.B = B;
  args.H = H;
  args.Hkv = Hkv;
  args.N = N;
  args.group = H / Hkv;
  args.c = (float)((double)scale * 1.4426950408889634);
  args.scale = scale;
  args.tiles = 0;
  args.total = 0;
  hipStream_t s = (hipStream_t)stream;
  return dtype == FA_DTYPE_BF16 ? dispatch_bwd<Bf16>(args, d, causal, s) : dispatch_bwd<F16>(args, d, causal, s);
}

}  // extern "C"
