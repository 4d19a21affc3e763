// fa_fwd.hip -- exact tiled attention forward for gfx950 (MI355X), and its C ABI.
//
// Method: the I/O-aware exact attention of "FlashAttention: Fast and Memory-Efficient
// Exact Attention with IO-Awareness" (abstract): key/value tiles stream through on-chip
// memory (here LDS), the scores of one tile live only in registers, and a running row
// maximum with a running exponential sum (section "What tiling changes" of "FlashAttention:
// The Algorithm That Made Long-Context AI Possible") replaces the full-row softmax, so the
// N x N matrix never reaches HBM. Work partitioning follows the abstract of
// "FlashAttention-2: Faster Attention with Better Parallelism and Work Partitioning":
// one workgroup per (batch, head, query tile) so that a single head still spreads over
// many CUs (item 2), and each wavefront owns disjoint query rows while sharing the
// workgroup's K/V tiles, so no partial output rows are reduced across wavefronts (item 3).
// Non-matmul work is kept small (item 1): the scale is folded into one FMA before a
// base-2 exponential, the output is normalised once at the end, and the accumulator is
// only rescaled when probabilities taken against the current maximum could overflow
// their 16-bit storage (a lane's sum above 2^15), not whenever the maximum grows.
//
// gfx950 mapping (one wavefront = 64 lanes, MFMA 32x32x16):
//   * The score tile is computed transposed, S^T = K Q^T, so that each lane holds one
//     query (lane % 32) and 16 keys per 32-key block: row max and row sum are lane-local
//     plus one v_permlane32_swap between lanes l and l^32.
//   * The output is accumulated transposed, O^T += V^T P^T, so the per-query rescale is
//     lane-local too. The probabilities leave the S^T accumulator already in the B-operand
//     layout of the next MFMA (keys are consumed in a permuted order, matched on the V side).
//   * K tiles go from global memory straight into LDS (buffer loads with an LDS
//     destination) in a 16-byte-chunk XOR swizzle; V tiles pass through registers, where
//     they are transposed into V^T (the transposing LDS read, ds_read_b64_tr_b16, runs at
//     a third of the rate of a plain read on gfx950).
//   * Each wavefront overlaps the MFMAs of the next score tile with the softmax of the
//     current one, and the P.V MFMAs with the staging of later tiles; K and V^T are
//     double-buffered in LDS, one barrier per key tile.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "fa.h"
#include "fa_env.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWaves = 8;              // wavefronts per workgroup (two per SIMD)
constexpr int kBr = 32 * kWaves;       // query rows per workgroup
constexpr int kBc = 64;                // keys per K/V tile
constexpr int kThreads = kWave * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// word 3 of a raw buffer descriptor on gfx9-family GPUs: 32-bit data format, no swizzle
constexpr int kBufferWord3 = 0x00020000;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Hkv, N;
  int group;            // H / Hkv
  int num_qtiles;       // ceil(N / kBr)
  int total;            // workgroups in the grid: num_qtiles * H * B
  float c;              // scale * log2(e) (times the q and k descales for e4m3)
  float v_scale;        // 1 for 16-bit inputs; the v descale for e4m3
  int wl, wr;           // key window of the band mask: query i sees keys i-wl .. i+wr
  // e4m3 with block scales: one E8M0 byte (2^(byte-127)) per FA_FP8_BLOCK_ROWS positions
  // of each (batch, head), [B][H][nb] for q and [B][Hkv][nb] for k and v
  const uint8_t* q_scales;
  const uint8_t* k_scales;
  const uint8_t* v_scales;
  int nb;
  // block-sparse mask: [mask_heads][nblk][nblk] bytes over blocks of kSparseBlock queries x
  // kSparseBlock keys, nonzero = computed; mask_heads is 1 (shared) or H
  const uint8_t* block_mask;
  int mask_heads, nblk;
};

// Masks, one kernel instance each: none; causal (key j visible to query i iff j <= i);
// band (iff i - wl <= j <= i + wr, the key window, which also covers a causal mask with
// a window: wr = 0).
constexpr int kMaskNone = 0;
constexpr int kMaskCausal = 1;
constexpr int kMaskBand = 2;
// block-sparse (iff the block mask keeps the (query block, key block) pair), alone or
// with the causal mask
constexpr int kMaskBlock = 3;
constexpr int kMaskBlockCausal = 4;             // block-sparse intersected with the causal mask
constexpr int kSparseBlock = 64;                // rows of a mask block, queries and keys
constexpr int kMaxSparseBlocks = 2048;          // key blocks per row of the mask: N <= 131072

// Workgroups are handed to the 8 XCDs round-robin (workgroup L runs on XCD L % 8), and
// each XCD has its own L2. Reorder so that XCD x receives one contiguous range of the
// logical work list, in which consecutive entries share K/V: the logical order is
// (batch, K/V head, query tile, query head within the group), query tiles longest first
// under a mask.
struct TileCoord {
  int b, h, qt;
};
__device__ __forceinline__ TileCoord tile_of_workgroup(const FwdArgs& a, int L, bool reverse) {
  const int xcd = L & 7, slot = L >> 3;
  const int per = a.total >> 3, rem = a.total & 7;
  const int logical = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int gm = logical % a.group;
  int t = logical / a.group;
  int qt = t % a.num_qtiles;
  t /= a.num_qtiles;
  const int hk = t % a.Hkv;
  const int b = t / a.Hkv;
  if (reverse) qt = a.num_qtiles - 1 - qt;
  return {b, hk * a.group + gm, qt};
}

// ---- element types ----------------------------------------------------------------
struct Bf16Ops {
  static constexpr float kPMax = 32768.0f;   // bound on stored probabilities (bf16 range is wider)
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float x, float y) {
    bf16x2 r = {(__bf16)x, (__bf16)y};  // v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(unsigned, r);
  }
};
struct F16Ops {
  static constexpr float kPMax = 32768.0f;   // below the largest finite f16, 65504
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float x, float y) {
    f16x2 r = {(_Float16)x, (_Float16)y};  // v_cvt_pk_f16_f32, round to nearest even
    return __builtin_bit_cast(unsigned, r);
  }
};

// ---- LDS tile layout ----------------------------------------------------------------
// K tile: kBc rows (keys) of D 16-bit elements, row-major like K in memory. Row r keeps
// its 16-byte chunks in XOR-permuted order, logical chunk c at physical c ^ kswz(r), so
// that 16 consecutive rows reading the same logical chunk hit 16 different bank groups.
//
// V tile: stored transposed as kBc/16 planes, one per group of 16 keys; plane g is D rows
// (dims) of the group's 16 keys, 32 bytes per row. Inside a row the keys are stored in the
// order in which a lane of the probability operand holds them: the lane with hi = lane/32
// holds keys {4hi..4hi+3, 8+4hi..8+4hi+3} of the group, which form the 16-byte chunk hi.
// The two chunks of row `dim` are swapped when bit 3 of dim is set, so that 16 lanes
// reading 16 consecutive rows cover all 64 banks once.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (D == 128) {
    const int x = r & 3;
    return ((x << 1) ^ (x << 2)) ^ ((r >> 2) & 3);
  } else {
    return r & 7;
  }
}

template <int D>
__device__ __forceinline__ int k_byte(int row, int col) {  // byte offset of K(row, col)
  return row * D * 2 + ((((col >> 3) ^ kswz<D>(row)) << 4) | ((col & 7) << 1));
}
// byte offset, inside a V^T tile, of chunk c (stored positions 8c..8c+7) of row `dim` in
// the plane of key group g
template <int D>
__device__ __forceinline__ int vt_byte(int g, int dim, int c) {
  return g * (D * 32) + dim * 32 + ((c ^ ((dim >> 3) & 1)) << 4);
}

// Maxima here use the NaN-propagating maximum (v_maximum3_f32 on gfx950): fmaxf's NaN
// rule makes the compiler quiet each MFMA result with an extra v_max before v_max3, while
// the two agree on every non-NaN input (masked scores are -inf, never NaN).
__device__ __forceinline__ float max_nan(float x, float y) { return __builtin_elementwise_maximum(x, y); }
__device__ __forceinline__ float pair_max(float x) {  // max over lanes l and l^32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {  // sum over lanes l and l^32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reductions over a lane's scores written as balanced trees: a single wavefront runs the
// softmax on its SIMD while the other issues MFMAs, so dependent-issue latency, not
// throughput, bounds these chains.
template <int KB>
__device__ __forceinline__ float tree_max(const f32x16 (&x)[KB]) {
  float t[KB * 16];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) t[kb * 16 + e] = x[kb][e];
  int n = KB * 16;
#pragma unroll
  for (int lvl = 0; lvl < 6; ++lvl) {
    if (n <= 1) break;
    int m = 0;
#pragma unroll
    for (int i = 0; i + 2 < n; i += 3) t[m++] = max_nan(max_nan(t[i], t[i + 1]), t[i + 2]);
    const int rem = n % 3;
    if (rem == 1) t[m++] = t[n - 1];
    if (rem == 2) t[m++] = max_nan(t[n - 2], t[n - 1]);
    n = m;
  }
  return t[0];
}
template <int KB>
__device__ __forceinline__ float tree_sum(const f32x16 (&x)[KB]) {
  float t[KB * 16];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) t[kb * 16 + e] = x[kb][e];
#pragma unroll
  for (int w = KB * 8; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = t[i] + t[i + w];
  return t[0];
}

typedef __attribute__((address_space(3))) unsigned char lds_byte;
template <typename T>
__device__ __forceinline__ T lds_load(const lds_byte* base, int byte_off) {
  return *(const __attribute__((address_space(3))) T*)(base + byte_off);
}
template <int V>
using ic = std::integral_constant<int, V>;

// ---- the forward kernel for 16-bit inputs -----------------------------------------------
// One workgroup of 8 wavefronts per (batch, head, 256-query tile); wavefront w owns query
// rows [32w, 32w+32) and all wavefronts share the K/V tiles staged in LDS. Each wavefront
// software-pipelines its own work: while the MFMAs of S(j+1) = K(j+1) Q^T run it computes
// the softmax of tile j, and while those of O^T += V^T(j) P^T(j) run it stages later tiles;
// one barrier per key tile hands the LDS buffers over.
// K tiles go from global memory straight into LDS (buffer loads with an LDS destination),
// so only V passes through registers, where it is transposed. K and V^T have two LDS
// slots each: during step j, K(j+2) goes to K slot j&1 and V(j+1) to V slot (j+1)&1, both
// after the barrier that ended the last read of that slot.
// s_waitcnt operand: vmcnt <= 8, expcnt and lgkmcnt not waited for
constexpr int kVmcnt8 = 0x8 | (0x7 << 4) | (0xF << 8);
// s_waitcnt operand: vmcnt <= 4, expcnt and lgkmcnt not waited for
constexpr int kVmcnt4 = 0x4 | (0x7 << 4) | (0xF << 8);

// one 16-byte-per-lane buffer load into LDS: lane i writes dst + 16 i
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, lds_byte* dst, unsigned voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voffset, 0, 0, 0);
}
// LDS address of a K-tile DMA destination, passed through an opaque register copy: the
// compiler then keeps no alias record of the DMA (it would otherwise wait for every DMA
// before every later LDS read), and the waits for it are the explicit vmcnt waits before
// the barriers of the kernel below
__device__ __forceinline__ lds_byte* lds_dma_dst(unsigned char* p) {
  unsigned v = (unsigned)(uintptr_t)(lds_byte*)p;
  asm volatile("" : "+s"(v));
  return (lds_byte*)(uintptr_t)v;
}

template <typename Ops, int D, int MASK>
__global__ __launch_bounds__(kThreads) void fa_fwd_overlap_kernel(FwdArgs a) {
  constexpr bool CAUSAL = MASK == kMaskCausal || MASK == kMaskBlockCausal;
  constexpr bool BAND = MASK == kMaskBand;
  constexpr bool BLOCKS = MASK == kMaskBlock || MASK == kMaskBlockCausal;
  static_assert(kSparseBlock == kBc && kBr % kSparseBlock == 0 && kBr / kSparseBlock <= 4, "mask blocks");
  constexpr int kChunks = D / 8;                  // 16-byte chunks per K row
  constexpr int kKsteps = D / 16;                 // MFMA k-steps over d for S^T
  constexpr int kDblocks = D / 32;                // 32-row blocks of O^T
  constexpr int kKb = kBc / 32;                   // 32-key blocks per tile
  constexpr int kTileBytes = kBc * D * 2;
  constexpr int kVBase = 2 * kTileBytes;

  // K slot 0, K slot 1, V^T slot 0, V^T slot 1
  __shared__ __attribute__((aligned(16))) unsigned char lds[4 * kTileBytes];
  // block-sparse: the workgroup's active key blocks, each entry kb | (q-block bits << 16),
  // then four entries -1 (past the end)
  __shared__ __attribute__((aligned(16))) int blk_list[BLOCKS ? kMaxSparseBlocks + 4 : 1];
  __shared__ int blk_count;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const TileCoord tc = tile_of_workgroup(a, blockIdx.x, MASK != kMaskNone);
  const int b = tc.b, h = tc.h, qt = tc.qt;
  const int hk = h / a.group;
  const int N = a.N;
  const int q0 = qt * kBr;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + l32;
  const int kv0 = BAND ? max(0, q0 - a.wl) / kBc * kBc : 0;
  const int nk = N - kv0;

  const size_t q_row_stride = (size_t)a.H * D;
  const size_t kv_row_stride = (size_t)a.Hkv * D;
  const uint16_t* qp = (const uint16_t*)a.q + ((size_t)b * N) * q_row_stride + (size_t)h * D;
  const uint16_t* kp = (const uint16_t*)a.k + ((size_t)b * N + kv0) * kv_row_stride + (size_t)hk * D;
  const uint16_t* vp = (const uint16_t*)a.v + ((size_t)b * N + kv0) * kv_row_stride + (size_t)hk * D;

  u32x4 qreg[kKsteps];
  const int qi_ld = min(qi, N - 1);
#pragma unroll
  for (int ks = 0; ks < kKsteps; ++ks)
    qreg[ks] = *(const u32x4*)(qp + (size_t)qi_ld * q_row_stride + ks * 16 + hi * 8);

  const int kv_end = BAND ? min(N, q0 + kBr + a.wr) : CAUSAL ? min(N, q0 + kBr) : N;
  // Block-sparse: wavefront 0 lists the key blocks that some query block of the workgroup
  // keeps (under the causal mask, only those up to the workgroup's last query), with the
  // query blocks that keep each (bit r: rows q0 + 64r ..); the tiles are these blocks.
  int nact = 0;
  if constexpr (BLOCKS) {
    const int nb = a.nblk, qb0 = q0 / kSparseBlock;
    const uint8_t* mrow = a.block_mask + ((size_t)(a.mask_heads == 1 ? 0 : h) * nb + qb0) * nb;
    const int kb_end = CAUSAL ? min(nb, (q0 + kBr) / kBc) : nb;
    if (wave == 0) {
      int count = 0;
      // every lane loads from a valid address (clamped to the mask) and discards what lies
      // outside it without a branch, so the four loads of an iteration go out together
      // rather than one per wait
      for (int base = 0; base < kb_end; base += kWave) {
        const int kb = base + lane;
        const int kbc = min(kb, nb - 1);
        int bits = 0;
#pragma unroll
        for (int r = 0; r < kBr / kSparseBlock; ++r) {
          const uint8_t v = mrow[(size_t)min(r, nb - 1 - qb0) * nb + kbc];
          bits |= (int)((kb < kb_end) & (qb0 + r < nb) & (v != 0)) << r;
        }
        const unsigned long long act = __ballot(bits != 0);
        if (bits) blk_list[count + __popcll(act & ((1ull << lane) - 1))] = kb | (bits << 16);
        count += __popcll(act);
      }
      if (lane == 0) blk_count = count;
      if (lane < 4) blk_list[count + lane] = -1;
    }
    __syncthreads();
    nact = blk_count;
  }
  const int ntiles = BLOCKS ? nact : (kv_end - kv0 + kBc - 1) / kBc;
  // Block-sparse: the list entry of tile j (-1 past the end, up to tile nact + 3) in a
  // uniform register. The loops below read the four entries of a pair of steps at once,
  // so that no list read waits among the operand reads of a step.
  auto tile_entry = [&](int j) __attribute__((always_inline)) {
    if constexpr (BLOCKS) return __builtin_amdgcn_readfirstlane(blk_list[j]);
    else return 0;
  };
  auto pair_entries = [&](int j, int (&e)[4]) __attribute__((always_inline)) {   // j even
    if constexpr (BLOCKS) {
      const int2 x = *(const int2*)&blk_list[j];
      const int2 y = *(const int2*)&blk_list[j + 2];
      e[0] = __builtin_amdgcn_readfirstlane(x.x);
      e[1] = __builtin_amdgcn_readfirstlane(x.y);
      e[2] = __builtin_amdgcn_readfirstlane(y.x);
      e[3] = __builtin_amdgcn_readfirstlane(y.y);
    } else {
      e[0] = e[1] = e[2] = e[3] = 0;
    }
  };
  // first key (relative to kv0) of tile j with list entry e; block-sparse tiles past the
  // list start at the end of the sequence, so their loads read zeros and their keys are
  // masked
  auto tile_k0 = [&](int j, int e) __attribute__((always_inline)) {
    if constexpr (BLOCKS) return e < 0 ? nk : (e & 0xffff) * kBc;
    else return j * kBc;
  };
  // whether this wavefront's query block keeps the tile with list entry e (block-sparse)
  auto tile_kept = [&](int e) __attribute__((always_inline)) {
    return e >= 0 && ((e >> (16 + (qw0 - q0) / kSparseBlock)) & 1) != 0;
  };

  int koff[kKsteps];
#pragma unroll
  for (int ks = 0; ks < kKsteps; ++ks) koff[ks] = k_byte<D>(l32, ks * 16 + hi * 8);
  int voff[kDblocks];
#pragma unroll
  for (int db = 0; db < kDblocks; ++db) voff[db] = kVBase + vt_byte<D>(0, db * 32 + l32, hi);

  // ---- staging ------------------------------------------------------------------------
  // Wavefront w stages keys [8w, 8w+8) of K and one V^T chunk of a tile:
  //   K: straight from global memory into LDS (buffer loads with an LDS destination, four
  //      rows of 1 KiB per instruction, lane i writing bytes 16i..16i+15 of them); the lane
  //      whose destination is chunk position c of row r loads logical chunk c ^ kswz(r),
  //      which gives the swizzled layout of k_byte;
  //   V: the 8 keys of stored chunk w&1 of key group w>>1, i.e. keys
  //      16(w>>1) + 4(w&1) + {0,1,2,3,8,9,10,11}; lane l loads dims 2l and 2l+1 of each
  //      (lanes past D/2 repeat the last pair) and transposes them into two V^T chunks.
  // Rows past the end of the sequence are read as zeros (the buffer descriptor's extent
  // is the sequence; their keys are masked), so no row index is clamped.
  constexpr int kKRows = kWave / kChunks;         // K rows per wavefront load
  constexpr int kKLoads = 8 / kKRows;             // K loads per lane per tile
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const unsigned row_bytes = (unsigned)(kv_row_stride * 2);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kp, 0, (int)(row_bytes * (unsigned)nk), kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vp, 0, (int)(row_bytes * (unsigned)nk), kBufferWord3);
  const int k_lane_row = lane / kChunks;
  unsigned k_lane_off[kKLoads];   // lane part of the K source offset of DMA u (row 8w + u kKRows + lane/kChunks)
#pragma unroll
  for (int u = 0; u < kKLoads; ++u)
    k_lane_off[u] = (unsigned)(k_lane_row * row_bytes) +
                    (unsigned)(((lane % kChunks) ^ kswz<D>(8 * wv + u * kKRows + k_lane_row)) * 16);
  const int vlane = min(lane, D / 2 - 1);
  const unsigned v_lane_off = (unsigned)vlane * 4u;
  unsigned vst[8];
  auto dma_k = [&](int k0, int slot) __attribute__((always_inline)) {   // k0: first key of the tile
#pragma unroll
    for (int u = 0; u < kKLoads; ++u) {
      const unsigned row0 = (unsigned)(k0 + 8 * wv + u * kKRows);
      lds_byte* dst = lds_dma_dst(lds + slot * kTileBytes + (8 * wv + u * kKRows) * D * 2);
      dma16(krs, dst, row0 * row_bytes + k_lane_off[u]);
    }
  };
  auto load_v = [&](int k0) __attribute__((always_inline)) {
    const unsigned r0 = (unsigned)(k0 + 16 * (wv >> 1) + 4 * (wv & 1));
#pragma unroll
    for (int r = 0; r < 8; ++r)
      vst[r] = __builtin_amdgcn_raw_buffer_load_b32(vrs, (r0 + (r & 3) + (r >> 2) * 8) * row_bytes + v_lane_off, 0, 0);
  };
  // V^T stores: store e writes, for each lane, dim 2l + ((e + bit 1 of l) & 1): then every
  // 8 consecutive lanes write 8 different 16-byte bank groups
  const unsigned v_sel_bit = (unsigned)((vlane >> 1) & 1);
  auto store_v = [&](int slot) __attribute__((always_inline)) {
    unsigned char* st = lds + kVBase + slot * kTileBytes;
    if (2 * lane < D) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const unsigned dd = (unsigned)e ^ v_sel_bit;
        const unsigned sel = dd ? 0x07060302u : 0x05040100u;
        u32x4 t;
#pragma unroll
        for (int q = 0; q < 4; ++q) t[q] = __builtin_amdgcn_perm(vst[2 * q + 1], vst[2 * q], sel);
        *(u32x4*)(st + vt_byte<D>(wv >> 1, 2 * lane + (int)dd, wv & 1)) = t;
      }
    }
  };

  // ---- per-wavefront state ------------------------------------------------------------
  f32x16 oacc[kDblocks];
#pragma unroll
  for (int i = 0; i < kDblocks; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.0f;
  f32x16 sA[kKb], sB[kKb];   // S^T of consecutive tiles alternate between these
  u32x4 p[kKb][2];
  // running max in base-2 exponent units (score * c); it starts at -FLT_MAX rather than
  // -inf so that a row whose keys in a tile are all masked gets exp2(-inf - m) = 0, never
  // exp2(-inf + inf)
  float m_run = -__FLT_MAX__;
  float l_run = 0.0f;        // this lane's part of the running denominator

  auto s_mfma = [&](f32x16 (&s)[kKb], int slot) __attribute__((always_inline)) {
    const lds_byte* st = (const lds_byte*)lds + slot * kTileBytes;
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kKsteps; ++ks)
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb)
        s[kb] = Ops::mfma(lds_load<u32x4>(st, koff[ks] + kb * 32 * D * 2), qreg[ks], s[kb]);
  };
  auto pv_mfma = [&](int slot) __attribute__((always_inline)) {
    const lds_byte* st = (const lds_byte*)lds + slot * kTileBytes;   // voff holds kVBase
#pragma unroll
    for (int kk = 0; kk < 2 * kKb; ++kk)
#pragma unroll
      for (int db = 0; db < kDblocks; ++db)
        oacc[db] = Ops::mfma(lds_load<u32x4>(st, voff[db] + kk * (D * 32)), p[kk >> 1][kk & 1], oacc[db]);
  };
  // masks the scores of the tile starting at key kv0 + k0r where some key of the tile is
  // invisible to some query of this wavefront (all of them for a tile the wavefront does
  // not see at all; KEPT is whether its query block keeps the tile, block-sparse)
  auto tile_needs_mask = [&](int k0r, bool kept) __attribute__((always_inline)) {
    const int k0 = kv0 + k0r;
    bool need = (k0 + kBc > N) || (CAUSAL && k0 + kBc - 1 > qw0);
    if constexpr (BAND) need = need || k0 + kBc - 1 > qw0 + a.wr || k0 < qw0 + 31 - a.wl;
    if constexpr (BLOCKS) need = need || !kept;
    return need;
  };
  auto mask_tile = [&](f32x16 (&s)[kKb], int k0r, bool kept) __attribute__((always_inline)) {
    const int k0 = kv0 + k0r;
    if (tile_needs_mask(k0r, kept)) {
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + kb * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
          bool dead = key >= N || (CAUSAL && key > qi) || (BLOCKS && !kept);
          if constexpr (BAND) dead = dead || key > qi + a.wr || key < qi - a.wl;
          s[kb][e] = dead ? -INFINITY : s[kb][e];
        }
    }
  };
  // Probabilities of a tile against the running maximum m_run as it stands, packed as the
  // B operand of P.V; returns this lane's sum of them. Every p is at most that sum, so while
  // the sum is <= Ops::kPMax no p can overflow the storage type of P and no rescale is
  // needed (exact in real arithmetic for any m_run). Otherwise a score grew past m_run by
  // more than log2(kPMax): the step below takes the tile's maximum, rescales the
  // accumulators and computes the probabilities again.
  auto exponentials = [&](const f32x16 (&s)[kKb]) __attribute__((always_inline)) {
    float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int e = hf * 8 + e2 * 2;
          const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], a.c, -m_run));
          const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e + 1], a.c, -m_run));
          part[e2] += x0 + x1;
          p[kb][hf][e2] = Ops::pack2(x0, x1);
        }
    return (part[0] + part[1]) + (part[2] + part[3]);
  };

  // S^T of tile j computed again from K in global memory (the rare path below: K slot j&1
  // may already hold K(j+2) from another wavefront). The operands are the ones staged to
  // LDS, so the scores are bit for bit the first ones, except for rows past the end of
  // the sequence (read here as row nk-1, there as zeros), whose keys are masked.
  auto s_global = [&](f32x16 (&s)[kKb], int k0r) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kKsteps; ++ks) {
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb) {
        const int key = min(k0r + kb * 32 + l32, nk - 1);
        const u32x4 ka = __builtin_amdgcn_raw_buffer_load_b128(krs, (unsigned)key * row_bytes + (unsigned)(ks * 16 + hi * 8) * 2u, 0, 0);
        s[kb] = Ops::mfma(ka, qreg[ks], s[kb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // raise m_run to cover the maximum of the tile's scores, rescaling O and l
  auto rescale_to = [&](const f32x16 (&s)[kKb]) __attribute__((always_inline)) {
    const float mx = pair_max(tree_max<kKb>(s)) * a.c;
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run = -FLT_MAX
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < kDblocks; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
  };

  // One step: the DMA of K(j+2), tile j's softmax beside S(j+1)'s MFMAs, then P(j).V(j)
  // beside the LDS stores of V(j+1) and the global loads of V(j+2); the caller then takes
  // the barrier. MASKED_C selects the body that masks tile j; a tile that needs no mask
  // skips the per-score compares and selects altogether.
  auto step = [&](f32x16 (&sc)[kKb], f32x16 (&sn)[kKb], auto par_c, int j, auto masked_c, int ej, int en)
      __attribute__((always_inline)) {   // ej, en: the list entries of tiles j and j+2
    constexpr int par = decltype(par_c)::value;   // j & 1
    constexpr bool kMasked = decltype(masked_c)::value;
    const int k0j = tile_k0(j, ej), k0n = tile_k0(j + 2, en);
    const bool kept = !BLOCKS || tile_kept(ej);
    dma_k(k0n, par);        // K slot j&1 was last read by S(j), before the previous barrier
    if constexpr (kMasked) mask_tile(sc, k0j, kept);
    // a row that has seen no visible key yet (m_run = -FLT_MAX) takes the tile's maximum
    // before its exponentials
    if (__builtin_amdgcn_ballot_w64(m_run == -__FLT_MAX__) != 0) rescale_to(sc);
    s_mfma(sn, par ^ 1);
    float lsum = exponentials(sc);
    // operand reads run kLead ahead of their MFMA; each MFMA is followed by 3 VALU
    // instructions of the softmax (measured best among 1-8), the rest after the last MFMA
    constexpr int kLead = 4;
    constexpr int kSOps = kKsteps * kKb;
    __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
    for (int i = 0; i < kSOps; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < kSOps - kLead) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
    if (__builtin_amdgcn_ballot_w64(!(lsum <= Ops::kPMax)) != 0) {
      // a score grew past m_run by more than log2(kPMax): the scores were consumed in
      // place, so they are computed again, then the tile's maximum and the probabilities
      f32x16 sr[kKb];
      s_global(sr, k0j);
      if constexpr (kMasked) mask_tile(sr, k0j, kept);
      rescale_to(sr);
      lsum = exponentials(sr);
    }
    l_run += lsum;
    pv_mfma(par);
    store_v(par ^ 1);
    load_v(k0n);
    // P.V operand reads kLeadB ahead (8 measured 0.3-0.7% faster than 4 or 6), the V
    // staging spread between the MFMAs
    constexpr int kPOps = kDblocks * 2 * kKb;
    constexpr int kLeadB = 8;
    __builtin_amdgcn_sched_group_barrier(0x100, kLeadB, 0);
#pragma unroll
    for (int i = 0; i < kPOps; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < kPOps - kLeadB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      if (i >= 8 && i < 12) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      if (i >= 8) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    // the K DMA of this step is complete (only the 8 V loads just issued may be pending)
    // before the barrier that publishes it
    __builtin_amdgcn_s_waitcnt(kVmcnt8);
  };

  // prologue: K(0), K(1) and V(0) in LDS, V(1) in registers, S(0) computed
  {
    const int k00 = tile_k0(0, tile_entry(0)), k01 = tile_k0(1, tile_entry(1));
    dma_k(k00, 0);
    dma_k(k01, 1);
    load_v(k00);
    store_v(0);
    load_v(k01);
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt8);
  __syncthreads();
  s_mfma(sA, 0);
  __syncthreads();   // every wavefront has read K slot 0 before K(2) replaces it

  // tiles go in pairs; an odd count gets one more tile, past kv_end, whose keys are all
  // masked for every query of the workgroup (probability 0)
  // Pairs of tiles that every wavefront of the workgroup sees whole (all keys in range
  // and, under the causal mask, at or before the workgroup's first query; under the band
  // mask, inside every query's band) run the unmasked body: a prefix of the loop for the
  // plain and causal masks, a middle range for the band, pairs chosen at run time
  // (uniformly for the workgroup) from the block-sparse list. The rest (the ragged end,
  // the causal diagonal, the band's edges, tiles some query block does not keep) run the
  // masked one. A choice per wavefront measured 2% slower than this uniform split.
  int j = 0;
  int e[4];
  if constexpr (BLOCKS) {
    // a listed tile is clear when every query block of the workgroup keeps it, it is whole
    // and, under the causal mask, it ends at or before the workgroup's first query
    const int qb_valid = min(kBr / kSparseBlock, a.nblk - q0 / kSparseBlock);
    const int all_bits = (1 << qb_valid) - 1;
    auto clear = [&](int ent) __attribute__((always_inline)) {
      const int k0 = (ent & 0xffff) * kBc;
      return ent >= 0 && ((ent >> 16) & all_bits) == all_bits && k0 + kBc <= N && (!CAUSAL || k0 + kBc - 1 <= q0);
    };
    // runs of clear pairs and of the other pairs alternate
    while (j < ntiles) {
      for (; j < ntiles; j += 2) {
        pair_entries(j, e);
        if (!(clear(e[0]) && clear(e[1]))) break;
        step(sA, sB, ic<0>(), j, std::false_type{}, e[0], e[2]);
        __syncthreads();
        step(sB, sA, ic<1>(), j + 1, std::false_type{}, e[1], e[3]);
        __syncthreads();
      }
      for (; j < ntiles; j += 2) {
        pair_entries(j, e);
        if (clear(e[0]) && clear(e[1])) break;
        step(sA, sB, ic<0>(), j, std::true_type{}, e[0], e[2]);
        __syncthreads();
        step(sB, sA, ic<1>(), j + 1, std::true_type{}, e[1], e[3]);
        __syncthreads();
      }
    }
  } else {
    pair_entries(0, e);
    // tile pairs [clear_begin, clear_end) run the unmasked body
    int clear_begin = 0, clear_end = 0;
    if constexpr (BAND) {
      // a tile is clear when its keys are in range and inside the band of every query of
      // the workgroup: first key >= the last query - wl, last key <= the first query + wr
      const int q_last = min(q0 + kBr, N) - 1;
      const int lo = q_last - a.wl - kv0;          // offsets from kv0
      const int hi = min(q0 + a.wr, N - 1) - kv0;
      const int jb = lo <= 0 ? 0 : (lo + kBc - 1) / kBc;
      const int je = hi < kBc - 1 ? 0 : (hi - (kBc - 1)) / kBc + 1;
      clear_begin = (jb + 1) & ~1;
      clear_end = max(clear_begin, je & ~1);
    } else {
      const int in_range = (N - kv0) / kBc;
      clear_end = (CAUSAL ? min(in_range, (q0 + 1 - kv0) / kBc) : in_range) & ~1;
    }
    for (; j < clear_begin; j += 2) {   // the band's left edge
      step(sA, sB, ic<0>(), j, std::true_type{}, e[0], e[2]);
      __syncthreads();
      step(sB, sA, ic<1>(), j + 1, std::true_type{}, e[1], e[3]);
      __syncthreads();
    }
    for (; j < clear_end; j += 2) {
      step(sA, sB, ic<0>(), j, std::false_type{}, e[0], e[2]);
      __syncthreads();
      step(sB, sA, ic<1>(), j + 1, std::false_type{}, e[1], e[3]);
      __syncthreads();
    }
    for (; j < ntiles; j += 2) {
      step(sA, sB, ic<0>(), j, std::true_type{}, e[0], e[2]);
      __syncthreads();
      step(sB, sA, ic<1>(), j + 1, std::true_type{}, e[1], e[3]);
      __syncthreads();
    }
  }

  // ---- epilogue -----------------------------------------------------------------------
  const float l_tot = pair_sum(l_run);
  if (qi < N) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;   // a row with no visible key: O = 0
    uint16_t* op = (uint16_t*)a.o + ((size_t)b * N + qi) * q_row_stride + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < kDblocks; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = db * 32 + g * 8 + hi * 4;
        u32x2 w;
        w[0] = Ops::pack2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
        w[1] = Ops::pack2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
        *(u32x2*)(op + dim) = w;
      }
    if (hi == 0) a.lse[((size_t)b * a.H + h) * N + qi] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

// ---- the forward kernel for OCP e4m3 inputs ----------------------------------------------
// The low-precision mode of "FlashAttention-3: Fast and Accurate Attention with Asynchrony
// and Low-precision" (abstract), with one descale per tensor: q, k, v are e4m3 codes whose
// values are multiplied by their tensor's descale. The online softmax is that of the 16-bit
// kernel, with three differences forced by gfx950's arithmetic:
//   * S^T = K Q^T runs on the bf16 MFMA after an exact e4m3 -> bf16 conversion (K while it
//     is staged, Q once): the e4m3 MFMAs sum each 64-term product with about 14 bits of
//     internal precision, which, with outlier elements, moves scores (and lse) by far more
//     than the bf16 path does;
//   * O^T += V^T P^T runs on v_mfma_f32_32x32x64_f8f6f4 with P stored as e4m3: its error
//     is relative to the output, well inside the e4m3 tolerance;
//   * P is taken against the running maximum shifted by kOff = 6 (p <= 2^(kTau+kOff) =
//     2^8.5 < 448), so that the bulk of the probabilities lands in e4m3's normal range, and
//     O is normalised by the sum of the stored probabilities (accumulated by the same MFMA
//     against an all-ones operand), which makes O a convex combination of V rows.
// P.V operands (lane l, hi = l/32, 32 bytes per lane): byte e of both operands is key
//   kfp8(hi, e) = 32(e/16) + 8((e%16)/4) + 4hi + e%4,
// the key of accumulator e%16 of S^T block e/16 held by that lane. V^T in LDS: rows (dims)
// of 64 bytes, byte 32hi + e holding V[kfp8(hi, e)][dim], chunks XOR-permuted by
// (dim >> 2) & 3.
// Schedule (ping-pong): the two halves of the workgroup (wavefronts 0-3 and 4-7, one of
// each per SIMD) run half a step apart, so that on every SIMD one wavefront issues MFMAs
// while the other computes the softmax. Step t (0 <= t < 2T+2, T key tiles) for a
// wavefront of half g: u = t - g; u even: MFMA block of j = u/2 (P.V of tile j-1, S of
// tile j); u odd: softmax block of tile j = u/2; every step ends with a workgroup barrier.
// Slot j (LDS buffer j&1, K tile then V^T tile) is read at steps 2j and 2j+1; its global
// loads go out at the end of step 2j-3 and it is written to LDS at the end of step 2j-1,
// after the last reader of slot j-2 (same buffer) has finished.
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_fp8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c) {
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  // formats 0/0: both operands e4m3; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// four e4m3 codes -> four bf16, times a power-of-two scale (exact: every e4m3 value is a
// bf16 value, and a power-of-two factor only moves the exponent)
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(unsigned x, float scale = 1.0f) {
  u32x2 r;
  r[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x, scale, false));
  r[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x, scale, true));
  return r;
}
// the same P.V product with operand A (V^T) scaled by an E8M0 byte (2^(byte-127)) per lane;
// every lane passes the same byte here, so the whole 64-key tile takes one scale
__device__ __forceinline__ f32x16 mfma_fp8_scaled(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c, int a_scale) {
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, a_scale, 0, 127);
}
// E8M0 byte -> float 2^(byte-127) (byte 0 is the subnormal 2^-127)
__device__ __forceinline__ float e8m0_to_f32(unsigned byte) {
  return __uint_as_float(byte ? byte << 23 : 0x00400000u);
}
// V^T tile of the e4m3 kernels in LDS: row dim of 64 bytes, 16-byte chunk c of a row at
// c ^ ((dim >> 2) & 3). The P.V operand reads (32 consecutive dims at one chunk) take the
// conflict-free time of a 16-byte read, as measured, and so do the 4-byte stores of the
// staging below, where each lane rotates which of its four dims it writes per store.
__device__ __forceinline__ int vt8q_byte(int dim, int pos) {
  return dim * 64 + ((((pos >> 4) ^ ((dim >> 2) & 3))) << 4) + (pos & 15);
}

template <int D, int MASK, bool BLOCK>
__global__ __launch_bounds__(kThreads) void fa_fwd_fp8_kernel(FwdArgs a) {
  constexpr bool CAUSAL = MASK == kMaskCausal;
  constexpr bool BAND = MASK == kMaskBand;
  constexpr float kTau = 2.5f;    // rescale once a row maximum grows by more than 2^kTau
  constexpr float kOff = 6.0f;    // probabilities are 2^kOff times softmax numerators
  constexpr int kKsteps = D / 16;                 // bf16 MFMA k-steps for S^T
  constexpr int kDblocks = D / 32;
  constexpr int kKb = kBc / 32;                   // 2 blocks of 32 keys
  constexpr int kTileK = kBc * D * 2;             // bf16 K tile in the layout of k_byte
  constexpr int kTileV = D * 64;                  // e4m3 V^T tile
  constexpr int kStageBytes = kTileK + kTileV;
  constexpr int kOnesBase = 2 * kStageBytes;      // 32 bytes of e4m3 ones, 32 of zeros: A operands of the probability sum
  static_assert(kBc == 64, "one P.V MFMA covers the 64 keys of a tile");

  __shared__ __attribute__((aligned(16))) unsigned char lds[kOnesBase + 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const TileCoord tc = tile_of_workgroup(a, blockIdx.x, MASK != kMaskNone);
  const int b = tc.b, h = tc.h, qt = tc.qt;
  const int hk = h / a.group;
  const int N = a.N;
  const int q0 = qt * kBr;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + l32;
  const int kv0 = BAND ? max(0, q0 - a.wl) / kBc * kBc : 0;   // as in the 16-bit kernel
  const int nk = N - kv0;
  const size_t q_row_stride = (size_t)a.H * D;    // bytes
  const size_t kv_row_stride = (size_t)a.Hkv * D;
  const uint8_t* qp = (const uint8_t*)a.q + ((size_t)b * N) * q_row_stride + (size_t)h * D;
  const uint8_t* kp = (const uint8_t*)a.k + ((size_t)b * N + kv0) * kv_row_stride + (size_t)hk * D;
  const uint8_t* vp = (const uint8_t*)a.v + ((size_t)b * N + kv0) * kv_row_stride + (size_t)hk * D;

  // Q^T operand in bf16: lane holds q[qi][16ks + 8hi .. +7]; with block scales the
  // wavefront's 32 queries lie in one block, whose scale the conversion applies exactly
  u32x4 qreg[kKsteps];
  const int qi_ld = min(qi, N - 1);
  float q_mult = 1.0f;
  if constexpr (BLOCK) q_mult = e8m0_to_f32(a.q_scales[((size_t)b * a.H + h) * a.nb + min(qw0, N - 1) / FA_FP8_BLOCK_ROWS]);
#pragma unroll
  for (int ks = 0; ks < kKsteps; ++ks) {
    const u32x2 raw = *(const u32x2*)(qp + (size_t)qi_ld * q_row_stride + ks * 16 + hi * 8);
    const u32x2 lo = e4m3x4_to_bf16(raw[0], q_mult), hi4 = e4m3x4_to_bf16(raw[1], q_mult);
    qreg[ks] = u32x4{lo[0], lo[1], hi4[0], hi4[1]};
  }

  const int kv_end = BAND ? min(N, q0 + kBr + a.wr) : CAUSAL ? min(N, q0 + kBr) : N;
  const int ntiles = (kv_end - kv0 + kBc - 1) / kBc;

  int koff[kKsteps];
#pragma unroll
  for (int ks = 0; ks < kKsteps; ++ks) koff[ks] = k_byte<D>(l32, ks * 16 + hi * 8);
  // P.V operand reads: dim 32 db + l32, bytes 32 hi + 16 x .. + 15 of its V^T row; the
  // chunk swizzle of a dim does not depend on db, so the blocks differ by 2 KiB
  int voff[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) voff[x] = kTileK + vt8q_byte(l32, hi * 32 + x * 16);
  constexpr int kVdbStride = 32 * kBc;

  // staging: wavefront w stages keys [8w, 8w+8) of K, and a quarter of V
  //   K: lane l -> key 8w + l/(D/16), 16 e4m3 codes (dims 16(l%(D/16)) ..), stored as bf16;
  //   V: the tile is 16 groups of 4 keys by D/64 halves of 64 dims. Wavefront w stages dim
  //      half w % (D/64) of four groups (set s = w / (D/64) < 4; wavefronts past 4 D/64 stage
  //      nothing): lane l takes group g = 8(s >> 1) + (s & 1) + 2(l & 3), whose keys lie in
  //      one 16-byte chunk of each V^T row at word l & 3, and dims 64 half + 4(l >> 2) .. + 3,
  //      a 4 x 4 byte transpose into four 4-byte V^T stores
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const unsigned row_bytes = (unsigned)kv_row_stride;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kp, 0, (int)(row_bytes * (unsigned)nk), kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vp, 0, (int)(row_bytes * (unsigned)nk), kBufferWord3);
  constexpr int kKLanes = 8 * (D / 16);           // lanes with 16 K codes
  const bool k_lane = lane < kKLanes;
  const int k_key = min(lane / (D / 16), 7), k_chunk = lane % (D / 16);
  constexpr int kVHalves = D / 64;
  const bool v_stager = 4 * kVHalves >= kWaves || wv < 4 * kVHalves;   // wavefront-uniform
  const int v_set = (wv / kVHalves) & 3, v_half = wv % kVHalves;
  const int v_grp = 8 * (v_set >> 1) + (v_set & 1) + 2 * (lane & 3);
  const int v_dq = lane >> 2;                     // dims 64 v_half + 4 v_dq .. + 3
  u32x4 kst;
  unsigned vst[4];
  // block scales of the staged tiles (key tile = scale block, both FA_FP8_BLOCK_ROWS = kBc
  // keys, and kv0 is a multiple of kBc): K's byte rides with its codes from load to store
  // and is applied by the conversion; V's becomes current when its tile is stored, and
  // stays so for both halves' P.V of that tile. The bytes are only read where the codes
  // are, so that no wait for the prefetch lands right after it is issued.
  static_assert(FA_FP8_BLOCK_ROWS == kBc, "one scale per key tile");
  const size_t kv_sc0 = ((size_t)b * a.Hkv + hk) * a.nb + kv0 / kBc;
  unsigned k_sc = 127;
  int v_sc_next = 127, v_sc = 127;
  auto load_k = [&](int j) __attribute__((always_inline)) {
    const int key = min(j * kBc + 8 * wv + k_key, nk - 1);
    kst = __builtin_amdgcn_raw_buffer_load_b128(krs, (unsigned)key * row_bytes + k_chunk * 16u, 0, 0);
    if constexpr (BLOCK) k_sc = a.k_scales[kv_sc0 + j];
  };
  // the row offset of a full tile is wavefront-uniform (scalar operand), the lane's group
  // rides in the per-lane offset; a ragged tile clamps rows per lane
  const unsigned v_col = (unsigned)(64 * v_half + 4 * v_dq);
  const unsigned v_lane_off = v_col + (unsigned)(4 * v_grp) * row_bytes;
  auto load_v = [&](int j) __attribute__((always_inline)) {
    const int j0 = j * kBc;
    if (v_stager) {
      if (j0 + kBc <= nk) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vst[r] = __builtin_amdgcn_raw_buffer_load_b32(vrs, v_lane_off, (j0 + r) * (int)row_bytes, 0);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = min(j0 + 4 * v_grp + r, nk - 1);
          vst[r] = __builtin_amdgcn_raw_buffer_load_b32(vrs, v_col + (unsigned)key * row_bytes, 0, 0);
        }
      }
    }
    if constexpr (BLOCK) v_sc_next = a.v_scales[kv_sc0 + j];
  };
  // The keys 4g .. 4g+3 of group g are bytes 32(g & 1) + 16(g >> 3) + 4((g >> 1) & 3) .. +3
  // of each V^T row (the key order of the P operand). Store t writes dim 4 v_dq + (t ^ rot),
  // rot = (v_dq >> 2) & 3: the first transpose stage takes each load's bytes in that order,
  // through per-lane byte selectors, and the address of store t is that of store 0 with bits
  // 6..7 flipped by t (the dim's low bits; the chunk swizzle is the same for the four dims,
  // and the tile bases are multiples of 256).
  const int v_rot = (v_dq >> 2) & 3;
  const int v_pos = 32 * (v_grp & 1) + 16 * (v_grp >> 3) + 4 * ((v_grp >> 1) & 3);
  const unsigned v_sel_lo = (unsigned)(v_rot | (4 + v_rot) << 8 | (v_rot ^ 1) << 16 | (4 + (v_rot ^ 1)) << 24);
  const int v_st0 = vt8q_byte(64 * v_half + 4 * v_dq + v_rot, v_pos);
  static_assert(kTileK % 256 == 0 && kStageBytes % 256 == 0, "V^T store addresses are formed by xor");
  auto store_k = [&](int buf) __attribute__((always_inline)) {
    if (!k_lane) return;
    const float k_mult = BLOCK ? e8m0_to_f32(k_sc) : 1.0f;
    unsigned char* st = lds + buf * kStageBytes;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const u32x2 c0 = e4m3x4_to_bf16(kst[2 * x], k_mult), c1 = e4m3x4_to_bf16(kst[2 * x + 1], k_mult);
      *(u32x4*)(st + k_byte<D>(8 * wv + k_key, k_chunk * 16 + x * 8)) = u32x4{c0[0], c0[1], c1[0], c1[1]};
    }
  };
  auto store_v = [&](int buf) __attribute__((always_inline)) {
    if constexpr (BLOCK) v_sc = v_sc_next;
    if (!v_stager) return;
    // 4x4 byte transpose: out[t] = bytes (key r = 0..3) of dim 4 v_dq + (t ^ rot)
    const unsigned v_sel_hi = v_sel_lo ^ 0x02020202u;        // dims rot ^ 2, rot ^ 3
    const unsigned t0 = __builtin_amdgcn_perm(vst[1], vst[0], v_sel_lo);
    const unsigned t1 = __builtin_amdgcn_perm(vst[1], vst[0], v_sel_hi);
    const unsigned t2 = __builtin_amdgcn_perm(vst[3], vst[2], v_sel_lo);
    const unsigned t3 = __builtin_amdgcn_perm(vst[3], vst[2], v_sel_hi);
    const unsigned out[4] = {__builtin_amdgcn_perm(t2, t0, 0x05040100u), __builtin_amdgcn_perm(t2, t0, 0x07060302u),
                             __builtin_amdgcn_perm(t3, t1, 0x05040100u), __builtin_amdgcn_perm(t3, t1, 0x07060302u)};
    unsigned char* vt = lds + buf * kStageBytes + kTileK;
#pragma unroll
    for (int t = 0; t < 4; ++t) *(unsigned*)(vt + (v_st0 ^ (64 * t))) = out[t];
  };

  f32x16 oacc[kDblocks];
#pragma unroll
  for (int i = 0; i < kDblocks; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.0f;
  f32x16 s[kKb];
  u32x4 p[2];                // 32 e4m3 probabilities: bytes e = 0..31 as in kfp8
  p[0] = u32x4{0u, 0u, 0u, 0u};
  p[1] = u32x4{0u, 0u, 0u, 0u};
  // sum of the stored probabilities, from a 16x16x128 MFMA of P against a 0/1 selector (as
  // in the kernel below, psum_mfma); every element holds the lane's sum
  f32x4 lacc;
#pragma unroll
  for (int e = 0; e < 4; ++e) lacc[e] = 0.0f;
  const u32x4 ones = {0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u};  // e4m3 1.0
  const int psel_off = kOnesBase + ((((lane >> 4) ^ (lane >> 2)) & 1) << 5);
  float m_run = -__FLT_MAX__;   // as in the 16-bit kernel
  float l_run = 0.0f;        // float32 sum of the unrounded probabilities (for lse)
  auto wave_active = [&](int j) __attribute__((always_inline)) {
    if constexpr (BAND) {
      const int k0 = kv0 + j * kBc;
      return j >= 0 && j < ntiles && k0 <= qw0 + 31 + a.wr && k0 + kBc - 1 >= qw0 - a.wl;
    } else {
      return !CAUSAL || j * kBc <= qw0 + 31;
    }
  };

  // In both parts the operand reads run ahead of their MFMAs in the source order (four K
  // reads; the V reads of two d-blocks), and a scheduling barrier after each MFMA keeps
  // that order; the scheduler otherwise put each read right before its MFMA.
  auto s_part = [&](const lds_byte* st) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.0f;
    constexpr int kN = kKsteps * kKb, kAhead = 4;
    u32x4 ka[kN];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) ka[i] = lds_load<u32x4>(st, koff[i / kKb] + (i % kKb) * 32 * D * 2);
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      if (i + kAhead < kN) ka[i + kAhead] = lds_load<u32x4>(st, koff[(i + kAhead) / kKb] + ((i + kAhead) % kKb) * 32 * D * 2);
      s[i % kKb] = Bf16Ops::mfma(ka[i], qreg[i / kKb], s[i % kKb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto pv_part = [&](const lds_byte* st) __attribute__((always_inline)) {
    u32x4 a0[kDblocks], a1[kDblocks];
#pragma unroll
    for (int db = 0; db < 2 && db < kDblocks; ++db) {
      a0[db] = lds_load<u32x4>(st, voff[0] + db * kVdbStride);
      a1[db] = lds_load<u32x4>(st, voff[1] + db * kVdbStride);
    }
#pragma unroll
    for (int db = 0; db < kDblocks; ++db) {
      if (db + 2 < kDblocks) {
        a0[db + 2] = lds_load<u32x4>(st, voff[0] + (db + 2) * kVdbStride);
        a1[db + 2] = lds_load<u32x4>(st, voff[1] + (db + 2) * kVdbStride);
      }
      if constexpr (BLOCK) oacc[db] = mfma_fp8_scaled(a0[db], a1[db], p[0], p[1], oacc[db], v_sc);
      else oacc[db] = mfma_fp8(a0[db], a1[db], p[0], p[1], oacc[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      const lds_byte* ob = (const lds_byte*)lds;
      const u32x4 s0 = lds_load<u32x4>(ob, psel_off), s1 = lds_load<u32x4>(ob, psel_off + 16);
      const i32x8 av = {(int)s0[0], (int)s0[1], (int)s0[2], (int)s0[3], (int)s1[0], (int)s1[1], (int)s1[2], (int)s1[3]};
      const i32x8 bv = {(int)p[0][0], (int)p[0][1], (int)p[0][2], (int)p[0][3], (int)p[1][0], (int)p[1][1], (int)p[1][2], (int)p[1][3]};
      lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, lacc, 0, 0, 0, 0, 0, 0);
    }
  };
  auto mfma_block = [&](auto buf_c, int j) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const lds_byte* st = (const lds_byte*)lds + buf * kStageBytes;
    if (j <= ntiles && (wave_active(j - 1) || (BAND && wave_active(j)))) {
      s_part(st);
      pv_part(st);
    }
  };
  auto softmax_block = [&](int j) __attribute__((always_inline)) {
    if (j >= ntiles || !wave_active(j)) return;
    const int k0 = kv0 + j * kBc;                  // first key of the tile
    bool need_mask = (k0 + kBc > N) || (CAUSAL && k0 + kBc - 1 > qw0);
    if constexpr (BAND) need_mask = need_mask || k0 + kBc - 1 > qw0 + a.wr || k0 < qw0 + 31 - a.wl;
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + kb * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
          bool dead = key >= N || (CAUSAL && key > qi);
          if constexpr (BAND) dead = dead || key > qi + a.wr || key < qi - a.wl;
          s[kb][e] = dead ? -INFINITY : s[kb][e];
        }
    }
    const float mx = pair_max(tree_max<kKb>(s)) * a.c;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kTau) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run = -FLT_MAX
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < kDblocks; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) lacc[e] *= alpha;
    }
    const float shift = kOff - m_run;
    f32x16 pe[kKb];
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) pe[kb][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], a.c, shift));
    // e4m3, round to nearest even: dword w of the operand holds bytes e = 4w .. 4w+3
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, i = (w & 3) * 4;
      int d = __builtin_amdgcn_cvt_pk_fp8_f32(pe[kb][i], pe[kb][i + 1], 0, false);
      d = __builtin_amdgcn_cvt_pk_fp8_f32(pe[kb][i + 2], pe[kb][i + 3], d, true);
      p[w >> 2][w & 3] = (unsigned)d;
    }
    l_run += tree_sum<kKb>(pe);
  };

  const int half = wv >> 2;
  load_k(0);
  store_k(0);
  {  // the V^T region of slot 0 (no tile -1) is zero, so step 0's P.V adds 0 * 0
    unsigned char* vz = lds + kTileK;
    for (int i = tid; i < kTileV / 16; i += kThreads) *(u32x4*)(vz + i * 16) = u32x4{0u, 0u, 0u, 0u};
    unsigned char* one = lds + kOnesBase;
    if (tid < 4) *(u32x4*)(one + tid * 16) = tid < 2 ? ones : u32x4{0u, 0u, 0u, 0u};
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (1 < ntiles) load_k(1);
  if (1 <= ntiles) load_v(0);
  __syncthreads();

  auto step = [&](auto phase_c, auto half_c, int t) __attribute__((always_inline)) {
    constexpr int phase = decltype(phase_c)::value;
    constexpr int hf = decltype(half_c)::value;
    if constexpr (hf == (phase & 1)) {
      mfma_block(ic<(phase >> 1) & 1>(), (t - hf) >> 1);
    } else {
      if (t - hf >= 0) softmax_block((t - hf) >> 1);
    }
    if constexpr ((phase & 1) == 1) {   // store slot jn, then load slot jn+1 (schedule above)
      const int jn = (t + 1) / 2;
      constexpr int buf = phase == 1 ? 1 : 0;
      if (jn < ntiles) store_k(buf);
      if (jn <= ntiles) store_v(buf);
      if (jn + 1 < ntiles) load_k(jn + 1);
      if (jn + 1 <= ntiles) load_v(jn);
    }
    __syncthreads();
  };
  auto run = [&](auto half_c) __attribute__((always_inline)) {
    const int nsteps = 2 * ntiles + 2;
    for (int t = 0; t < nsteps; t += 4) {
      step(ic<0>(), half_c, t);
      step(ic<1>(), half_c, t + 1);
      step(ic<2>(), half_c, t + 2);
      step(ic<3>(), half_c, t + 3);
    }
  };
  if (half == 0) run(ic<0>());
  else run(ic<1>());

  // epilogue: O = O_acc * v_descale / (sum of stored probabilities) in bf16; lse from the
  // float32 sum of the unrounded probabilities, undoing the 2^kOff shift
  const float l_tot = pair_sum(l_run);
  if (qi < N) {
    const float inv = a.v_scale / lacc[0];
    uint16_t* op = (uint16_t*)a.o + ((size_t)b * N + qi) * ((size_t)a.H * D) + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < kDblocks; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = db * 32 + g * 8 + hi * 4;
        u32x2 w;
        w[0] = Bf16Ops::pack2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
        w[1] = Bf16Ops::pack2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
        *(u32x2*)(op + dim) = w;
      }
    if (hi == 0) a.lse[((size_t)b * a.H + h) * N + qi] = (m_run - kOff + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

// ---- the forward kernel for e4m3 inputs on fp8 MFMAs -----------------------------------
// Both products on the e4m3 MFMA v_mfma_scale_f32_32x32x64_f8f6f4 (four times the bf16
// MFMA's k per instruction, at the same cycle count per 32 x 32 output block):
//   * S^T = K Q^T: A = a K tile row (64 dims of one key, 32 bytes per lane), B = the Q row
//     (the same 64 dims of one query); any pairing of dims between A and B bytes gives the
//     same sum, so each lane holds 32 consecutive bytes of its row. Q and K block scales
//     (E8M0) go into the instruction's scale operands and are applied exactly;
//   * O^T += V^T P^T as in the kernel above (one MFMA per 32 dims covers the tile's 64 keys),
//     with the sum of the stored probabilities from one 16x16x128 e4m3 MFMA of P against a
//     0/1 selector (half the cycles of a 32x32x64 one, four accumulator registers).
// K tiles go from global memory straight into LDS (LDS DMA) as e4m3 bytes; V passes through
// registers and is transposed into V^T there (4 x 4 byte transposes). The workgroup and
// schedule follow the 16-bit kernel: 8 wavefronts of 32 query rows in lockstep, two K and two
// V^T slots, one barrier per key tile. Because one P.V MFMA consumes all 64 keys of P, P.V
// of tile j is deferred to step j+1, where it runs beside the MFMAs of S(j+2) and the softmax
// of tile j+1, so the softmax is spread over all the MFMAs of a step.
// The running maximum moves only when a tile's maximum exceeds it by more than kTau (the
// maximum is taken in the step before the tile's exponentials); probabilities are stored as
// e4m3 times 2^kOff, p <= 2^(kTau + kOff) = 2^8.5 < 448, so the bulk of them lies in
// e4m3's normal range. O is normalised by the sum of the stored probabilities (O is a
// convex combination of V rows); lse uses the float32 sum of the unrounded ones.
// K tile in LDS: row r (key) of D bytes, 16-byte chunk c at c ^ k8swz(r). Any 8
// consecutive rows read at one logical chunk hit 8 different 16-byte units of a 128-byte
// bank window, and any 16 consecutive rows 16 different units of a 256-byte window, so the
// S^T operand reads are free of bank conflicts whether the LDS serves 8 or 16 lanes of a
// 16-byte read per cycle.
template <int D>
__device__ __forceinline__ int k8swz(int r) {
  if constexpr (D == 128) return (r ^ ((r >> 3) & 3)) & 7;
  else return ((((r >> 2) ^ (r >> 3)) & 1) << 1) | (((r >> 1) ^ (r >> 3)) & 1);
}
constexpr int kMaxScaleTiles = 2048;            // block-scaled e4m3: N <= 131072

template <int D, int MASK, bool BLOCK>
__global__ __launch_bounds__(kThreads) void fa_fwd_e4m3qk_kernel(FwdArgs a) {
  constexpr bool CAUSAL = MASK == kMaskCausal;
  constexpr bool BAND = MASK == kMaskBand;
  constexpr float kTau = 2.5f;
  constexpr float kOff = 6.0f;
  constexpr int kKsteps = D / 64;                 // 64-dim k-steps of S^T
  constexpr int kDblocks = D / 32;                // 32-row blocks of O^T
  constexpr int kKb = kBc / 32;                   // 32-key blocks per tile
  constexpr int kChunks = D / 16;                 // 16-byte chunks per K row
  constexpr int kTileK = kBc * D;                 // e4m3 K tile
  constexpr int kTileV = D * kBc;                 // e4m3 V^T tile
  constexpr int kVBase = 2 * kTileK;
  constexpr int kOnesBase = kVBase + 2 * kTileV;  // 32 bytes of e4m3 ones, 32 of zeros: A operands of the probability sum
  constexpr int kSOps = kKsteps * kKb;            // S^T MFMAs per tile
  static_assert(kBc == 64 && FA_FP8_BLOCK_ROWS == kBc, "one P.V MFMA and one block scale per key tile");

  // K slot 0, K slot 1, V^T slot 0, V^T slot 1, ones
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kTileK + 2 * kTileV + 64];
  // block scales of the K and V tiles of this (batch, K/V head), two entries of 127 (2^0)
  // past the end
  __shared__ unsigned char kscale[BLOCK ? kMaxScaleTiles + 4 : 1];
  __shared__ unsigned char vscale[BLOCK ? kMaxScaleTiles + 4 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const TileCoord tc = tile_of_workgroup(a, blockIdx.x, MASK != kMaskNone);
  const int b = tc.b, h = tc.h, qt = tc.qt;
  const int hk = h / a.group;
  const int N = a.N;
  const int q0 = qt * kBr;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + l32;
  const int kv0 = BAND ? max(0, q0 - a.wl) / kBc * kBc : 0;
  const int nk = N - kv0;
  const size_t q_row_stride = (size_t)a.H * D;    // bytes
  const size_t kv_row_stride = (size_t)a.Hkv * D;
  const uint8_t* qp = (const uint8_t*)a.q + ((size_t)b * N) * q_row_stride + (size_t)h * D;
  const uint8_t* kp = (const uint8_t*)a.k + ((size_t)b * N + kv0) * kv_row_stride + (size_t)hk * D;
  const uint8_t* vp = (const uint8_t*)a.v + ((size_t)b * N + kv0) * kv_row_stride + (size_t)hk * D;

  // Q^T operand: lane holds q[qi][64 ks + 32 hi .. + 31] for k-step ks. The wavefront's 32
  // queries lie in one scale block.
  const int qi_ld = min(qi, N - 1);
  int q_sc = 0;
  if constexpr (BLOCK) q_sc = a.q_scales[((size_t)b * a.H + h) * a.nb + min(qw0, N - 1) / FA_FP8_BLOCK_ROWS];
  i32x8 qreg[kKsteps];
#pragma unroll
  for (int ks = 0; ks < kKsteps; ++ks) {
    const u32x4 x0 = *(const u32x4*)(qp + (size_t)qi_ld * q_row_stride + ks * 64 + hi * 32);
    const u32x4 x1 = *(const u32x4*)(qp + (size_t)qi_ld * q_row_stride + ks * 64 + hi * 32 + 16);
    qreg[ks] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  }

  const int kv_end = BAND ? min(N, q0 + kBr + a.wr) : CAUSAL ? min(N, q0 + kBr) : N;
  const int ntiles = (kv_end - kv0 + kBc - 1) / kBc;
  if constexpr (BLOCK) {
    const size_t sc0 = ((size_t)b * a.Hkv + hk) * a.nb + kv0 / kBc;
    for (int t = tid; t < ntiles + 4; t += kThreads) {
      const bool in = t < ntiles && kv0 / kBc + t < a.nb;
      kscale[t] = in ? a.k_scales[sc0 + t] : (unsigned char)127;
      vscale[t] = in ? a.v_scales[sc0 + t] : (unsigned char)127;
    }
  }

  // S^T operand reads: key l32 of 32-key block kb, chunks 4 ks + 2 hi and + 1
  int koff[kKsteps][2];
#pragma unroll
  for (int ks = 0; ks < kKsteps; ++ks)
#pragma unroll
    for (int x = 0; x < 2; ++x) koff[ks][x] = l32 * D + (((4 * ks + 2 * hi + x) ^ k8swz<D>(l32)) << 4);
  constexpr int kKbStride = 32 * D;               // bytes between the 32-key blocks of a K tile
  // P.V operand reads: dim 32 db + l32, bytes 32 hi + 16 x .. + 15; the chunk swizzle of a
  // dim does not depend on db (bits 1.. 3 of 32 db are zero), so blocks differ by 2 KiB
  int voff[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) voff[x] = kVBase + vt8q_byte(l32, hi * 32 + x * 16);
  constexpr int kVdbStride = 32 * kBc;

  // ---- staging ------------------------------------------------------------------------
  //   K: kTileK / 1 KiB DMA instructions per tile, one per wavefront w < kTileK / 1024; lane
  //      i writes row 1024 w / D + i / kChunks at chunk position i % kChunks and loads the
  //      logical chunk that position holds (rows past the end of the sequence read zeros);
  //   V: the tile is 16 groups of 4 keys by D/64 halves of 64 dims. Wavefront w stages dim
  //      half w % (D/64) of four groups (set s = w / (D/64) < 4; wavefronts past 4 D/64 stage
  //      nothing): lane l takes group g = 8(s >> 1) + (s & 1) + 2(l & 3), whose keys lie in
  //      one 16-byte chunk of each V^T row at word l & 3, and dims 64 half + 4(l >> 2) .. + 3.
  //      A 4 x 4 byte transpose turns its four 4-byte loads into four 4-byte V^T stores; rows
  //      past the end of the sequence read as zeros (their keys are masked).
  constexpr int kKDma = kTileK / 1024;
  constexpr int kKRowsPerDma = 1024 / D;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const unsigned row_bytes = (unsigned)kv_row_stride;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kp, 0, (int)(row_bytes * (unsigned)nk), kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vp, 0, (int)(row_bytes * (unsigned)nk), kBufferWord3);
  const int k_row_in_dma = lane / kChunks;
  const unsigned k_lane_off = (unsigned)(k_row_in_dma * row_bytes) +
      (unsigned)(((lane % kChunks) ^ k8swz<D>(kKRowsPerDma * wv + k_row_in_dma)) * 16);
  auto dma_k = [&](int k0, int slot) __attribute__((always_inline)) {   // k0: first key of the tile
    if constexpr (kKDma < kWaves) {
      if (wv >= kKDma) return;
    }
    const unsigned row0 = (unsigned)(k0 + kKRowsPerDma * wv);
    lds_byte* dst = lds_dma_dst(lds + slot * kTileK + kKRowsPerDma * wv * D);
    dma16(krs, dst, row0 * row_bytes + k_lane_off);
  };
  constexpr int kVHalves = D / 64;
  const bool v_stager = 4 * kVHalves >= kWaves || wv < 4 * kVHalves;   // wavefront-uniform
  const int v_set = (wv / kVHalves) & 3, v_half = wv % kVHalves;
  const int v_grp = 8 * (v_set >> 1) + (v_set & 1) + 2 * (lane & 3);
  const int v_dq = lane >> 2;                     // dims 64 v_half + 4 v_dq .. + 3
  const unsigned v_lane_off = (unsigned)(64 * v_half + 4 * v_dq) + (unsigned)(4 * v_grp) * row_bytes;
  unsigned vst[4];
  auto load_v = [&](int k0) __attribute__((always_inline)) {
    if (!v_stager) return;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      vst[r] = __builtin_amdgcn_raw_buffer_load_b32(vrs, (unsigned)(k0 + r) * row_bytes + v_lane_off, 0, 0);
  };
  // The keys 4g .. 4g+3 of group g are bytes 32(g & 1) + 16(g >> 3) + 4((g >> 1) & 3) .. +3
  // of each V^T row (the key order of the P operand). Store t writes dim 4 v_dq + (t ^ rot),
  // rot = (v_dq >> 2) & 3: the first transpose stage takes each load's bytes in that order,
  // through per-lane byte selectors, and the address of store t is that of store 0 with bits
  // 6..7 flipped by t (the dim's low bits; the chunk swizzle is the same for the four dims,
  // and the tile bases are multiples of 256).
  const int v_rot = (v_dq >> 2) & 3;
  const int v_pos = 32 * (v_grp & 1) + 16 * (v_grp >> 3) + 4 * ((v_grp >> 1) & 3);
  const unsigned v_sel_lo = (unsigned)(v_rot | (4 + v_rot) << 8 | (v_rot ^ 1) << 16 | (4 + (v_rot ^ 1)) << 24);
  const int v_st0 = vt8q_byte(64 * v_half + 4 * v_dq + v_rot, v_pos);
  static_assert(kVBase % 256 == 0 && kTileV % 256 == 0, "V^T store addresses are formed by xor");
  auto store_v = [&](int slot) __attribute__((always_inline)) {
    if (!v_stager) return;
    // 4x4 byte transpose: out[t] = bytes (key r = 0..3) of dim 4 v_dq + (t ^ rot)
    const unsigned v_sel_hi = v_sel_lo ^ 0x02020202u;        // dims rot ^ 2, rot ^ 3
    const unsigned t0 = __builtin_amdgcn_perm(vst[1], vst[0], v_sel_lo);
    const unsigned t1 = __builtin_amdgcn_perm(vst[1], vst[0], v_sel_hi);
    const unsigned t2 = __builtin_amdgcn_perm(vst[3], vst[2], v_sel_lo);
    const unsigned t3 = __builtin_amdgcn_perm(vst[3], vst[2], v_sel_hi);
    const unsigned out[4] = {__builtin_amdgcn_perm(t2, t0, 0x05040100u), __builtin_amdgcn_perm(t2, t0, 0x07060302u),
                             __builtin_amdgcn_perm(t3, t1, 0x05040100u), __builtin_amdgcn_perm(t3, t1, 0x07060302u)};
    unsigned char* vt = lds + kVBase + slot * kTileV;
#pragma unroll
    for (int t = 0; t < 4; ++t) *(unsigned*)(vt + (v_st0 ^ (64 * t))) = out[t];
  };

  // ---- per-wavefront state ------------------------------------------------------------
  f32x16 oacc[kDblocks];
#pragma unroll
  for (int i = 0; i < kDblocks; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.0f;
  f32x4 lacc;        // sum of the stored probabilities (every element holds the lane's sum)
#pragma unroll
  for (int e = 0; e < 4; ++e) lacc[e] = 0.0f;
  f32x16 sA[kKb], sB[kKb];
  u32x4 pc[2], pn[2];        // e4m3 probabilities of the tile whose P.V is pending, and of the next
  pc[0] = pc[1] = pn[0] = pn[1] = u32x4{0u, 0u, 0u, 0u};
  const u32x4 ones = {0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u};  // e4m3 1.0
  // The probability sum runs on a 16x16x128 MFMA. Its B operand is the P operand itself:
  // lane l (k-group G = l >> 4, column l & 15) holds the keys of query l & 31 from half l >> 5,
  // so k-groups G and G ^ 2 of column n belong to query n + 16 (G & 1). The A operand selects
  // k-group G for the output rows m with (m >> 2) & 1 == G & 1 (A lane l: row l & 15, k-group
  // l >> 4, all ones or all zeros), which puts the sum of query l & 31 in the four outputs of
  // lane l. Both kinds of A operand are read from LDS (32 bytes of ones, then 32 of zeros).
  const int psel_off = kOnesBase + ((((lane >> 4) ^ (lane >> 2)) & 1) << 5);
  auto psum_mfma = [&](const u32x4 (&pp)[2], const f32x4& c) __attribute__((always_inline)) {
    const lds_byte* ob = (const lds_byte*)lds;
    const u32x4 a0 = lds_load<u32x4>(ob, psel_off), a1 = lds_load<u32x4>(ob, psel_off + 16);
    const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8 bv = {(int)pp[0][0], (int)pp[0][1], (int)pp[0][2], (int)pp[0][3],
                      (int)pp[1][0], (int)pp[1][1], (int)pp[1][2], (int)pp[1][3]};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
  };
  float m_run = -__FLT_MAX__;
  float l_run = 0.0f;        // float32 sum of the unrounded probabilities (for lse)
  float mx_cur;              // maximum of the tile whose exponentials come next

  // S^T MFMA i (k-step i / kKb, 32-key block i % kKb) on the K slot at ks_
  auto s_op = [&](const lds_byte* ks_, int i, const f32x16& c, int k_sc) __attribute__((always_inline)) {
    const int ks = i / kKb, kb = i % kKb;
    const u32x4 a0 = lds_load<u32x4>(ks_, koff[ks][0] + kb * kKbStride);
    const u32x4 a1 = lds_load<u32x4>(ks_, koff[ks][1] + kb * kKbStride);
    const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    if constexpr (BLOCK) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qreg[ks], c, 0, 0, 0, k_sc, 0, q_sc);
    else return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qreg[ks], c, 0, 0, 0, 0, 0, 0);
  };
  auto pv_mfma = [&](const u32x4& a0, const u32x4& a1, const u32x4 (&pp)[2], const f32x16& c, int v_sc)
      __attribute__((always_inline)) {
    if constexpr (BLOCK) return mfma_fp8_scaled(a0, a1, pp[0], pp[1], c, v_sc);
    else return mfma_fp8(a0, a1, pp[0], pp[1], c);
  };
  auto tile_needs_mask = [&](int k0r) __attribute__((always_inline)) {
    const int k0 = kv0 + k0r;
    bool need = (k0 + kBc > N) || (CAUSAL && k0 + kBc - 1 > qw0);
    if constexpr (BAND) need = need || k0 + kBc - 1 > qw0 + a.wr || k0 < qw0 + 31 - a.wl;
    return need;
  };
  auto mask_tile = [&](f32x16 (&s)[kKb], int k0r) __attribute__((always_inline)) {
    const int k0 = kv0 + k0r;
    if (tile_needs_mask(k0r)) {
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + kb * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
          bool dead = key >= N || (CAUSAL && key > qi);
          if constexpr (BAND) dead = dead || key > qi + a.wr || key < qi - a.wl;
          s[kb][e] = dead ? -INFINITY : s[kb][e];
        }
    }
  };
  auto tile_max = [&](const f32x16 (&s)[kKb]) __attribute__((always_inline)) {
    return pair_max(tree_max<kKb>(s)) * a.c;
  };
  // exponentials of a tile in place (float32, for lse) and their e4m3 codes into pn: dword w
  // of the operand holds bytes e = 4w .. 4w+3 (key order of the S^T accumulator)
  auto exponentials = [&](f32x16 (&s)[kKb]) __attribute__((always_inline)) {
    const float shift = kOff - m_run;
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], a.c, shift));
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, i = (w & 3) * 4;
      // both halves are written: the previous word only fills the operand
      int d = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][i], s[kb][i + 1], (int)pn[w >> 2][w & 3], false);
      d = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][i + 2], s[kb][i + 3], d, true);
      pn[w >> 2][w & 3] = (unsigned)d;
    }
  };
  // P.V and the probability sum of the pending tile (V^T slot vslot, V scale v_sc)
  auto pending_pv = [&](int vslot, int v_sc) __attribute__((always_inline)) {
    const lds_byte* vs_ = (const lds_byte*)lds + vslot * kTileV;   // voff holds kVBase
#pragma unroll
    for (int db = 0; db < kDblocks; ++db)
      oacc[db] = pv_mfma(lds_load<u32x4>(vs_, voff[0] + db * kVdbStride), lds_load<u32x4>(vs_, voff[1] + db * kVdbStride), pc, oacc[db], v_sc);
    lacc = psum_mfma(pc, lacc);
  };

  // One step, for tile j (scores S(j) in sc, maximum mx_cur): the rescale decision for tile
  // j (the rare path first adds the pending P(j-1).V(j-1) under the old maximum and clears
  // P(j-1)), then one scheduling region: the MFMAs of S(j+1) = K(j+1) Q^T, then those of
  // P(j-1).V(j-1) and its sum, beside the exponentials and e4m3 packing of P(j), its float32
  // row sum, the mask (MASKED_C: whether tile j+1 needs one) and maximum of S(j+1), the LDS
  // stores of V(j) and the global loads of V(j+1). The DMA of K(j+2) goes out first.
  auto step = [&](f32x16 (&sc)[kKb], f32x16 (&sn)[kKb], auto par_c, int j, auto masked_c)
      __attribute__((always_inline)) {
    constexpr int par = decltype(par_c)::value;   // j & 1
    constexpr bool kMasked = decltype(masked_c)::value;
    dma_k((j + 2) * kBc, par);   // K slot j&1 was last read by S(j), before the previous barrier
    const int k_sc = BLOCK ? (int)kscale[j + 1] : 0;
    const int v_sc = BLOCK ? (int)vscale[max(j - 1, 0)] : 0;
    if (__builtin_amdgcn_ballot_w64(mx_cur > m_run + kTau) != 0) {
      pending_pv(par ^ 1, v_sc);
      pc[0] = pc[1] = u32x4{0u, 0u, 0u, 0u};
      const float m_new = fmaxf(m_run, mx_cur);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run = -FLT_MAX
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < kDblocks; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) lacc[e] *= alpha;
    }
    const lds_byte* ks_ = (const lds_byte*)lds + (par ^ 1) * kTileK;
    const lds_byte* vs_ = (const lds_byte*)lds + (par ^ 1) * kTileV;    // V^T of tile j-1; voff holds kVBase
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sn[kb][e] = 0.0f;
#pragma unroll
    for (int i = 0; i < kSOps; ++i) sn[i % kKb] = s_op(ks_, i, sn[i % kKb], k_sc);
    exponentials(sc);
#pragma unroll
    for (int db = 0; db < kDblocks; ++db)
      oacc[db] = pv_mfma(lds_load<u32x4>(vs_, voff[0] + db * kVdbStride), lds_load<u32x4>(vs_, voff[1] + db * kVdbStride), pc, oacc[db], v_sc);
    lacc = psum_mfma(pc, lacc);
    l_run += tree_sum<kKb>(sc);
    if constexpr (kMasked) mask_tile(sn, (j + 1) * kBc);
    mx_cur = tile_max(sn);
    store_v(par);
    load_v((j + 1) * kBc);
    pc[0] = pn[0];
    pc[1] = pn[1];
    // MFMAs in program order, the operand reads two MFMAs ahead, the VALU work spread
    // between them
    constexpr int kSReads = 2;                     // LDS operand reads per S^T MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kSReads, 0);
#pragma unroll
    for (int i = 0; i < kSOps; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, kSReads, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 80 / kSOps, 0);
    }
#pragma unroll
    for (int i = 0; i < kDblocks + 1; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < kDblocks - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 70 / (kDblocks + 1), 0);
    }
    // the K DMA of this step is complete (only the V loads just issued may be pending)
    // before the barrier that publishes it
    __builtin_amdgcn_s_waitcnt(kVmcnt4);
  };

  // prologue: K(0), K(1) in LDS, V(0) in registers, the V^T slot of the (absent) tile -1
  // zero, S(0) computed, masked and its maximum taken
  dma_k(0, 0);
  dma_k(kBc, 1);
  load_v(0);
  {
    unsigned char* vz = lds + kVBase + kTileV;   // slot 1: read by step 0 with P = 0
    for (int i = tid; i < kTileV / 16; i += kThreads) *(u32x4*)(vz + i * 16) = u32x4{0u, 0u, 0u, 0u};
    unsigned char* one = lds + kOnesBase;
    if (tid < 4) *(u32x4*)(one + tid * 16) = tid < 2 ? ones : u32x4{0u, 0u, 0u, 0u};
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt4);
  __syncthreads();
  {
    const int k_sc0 = BLOCK ? (int)kscale[0] : 0;
    const lds_byte* ks_ = (const lds_byte*)lds;
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sA[kb][e] = 0.0f;
#pragma unroll
    for (int i = 0; i < kSOps; ++i) sA[i % kKb] = s_op(ks_, i, sA[i % kKb], k_sc0);
    mask_tile(sA, 0);
    mx_cur = tile_max(sA);
  }
  __syncthreads();   // every wavefront has read K slot 0 before K(2) replaces it

  // Tiles go in pairs of steps (an odd count gets one more, fully masked tile). Step j masks
  // tile j+1: a pair (j, j+1) runs the unmasked body while tiles j+1 and j+2 are seen whole
  // by every wavefront (in range and, under the causal mask, at or before the workgroup's
  // first query), a prefix of the loop; the rest runs the masked body.
  int clear_tiles = 0;
  if constexpr (!BAND) {
    const int in_range = (N - kv0) / kBc;
    clear_tiles = CAUSAL ? min(in_range, (q0 + 1 - kv0) / kBc) : in_range;
  }
  int j = 0;
  for (; j + 2 < clear_tiles; j += 2) {
    step(sA, sB, ic<0>(), j, std::false_type{});
    __syncthreads();
    step(sB, sA, ic<1>(), j + 1, std::false_type{});
    __syncthreads();
  }
  for (; j < ntiles; j += 2) {
    step(sA, sB, ic<0>(), j, std::true_type{});
    __syncthreads();
    step(sB, sA, ic<1>(), j + 1, std::true_type{});
    __syncthreads();
  }
  // the last tile's P.V (its V^T was stored by the last step, before its barrier)
  pending_pv((j - 1) & 1, BLOCK ? (int)vscale[j - 1] : 0);

  // epilogue: O = O_acc * v_descale / (sum of stored probabilities) in bf16; lse from the
  // float32 sum of the unrounded probabilities, undoing the 2^kOff shift
  const float l_tot = pair_sum(l_run);
  if (qi < N) {
    const float inv = lacc[0] > 0.0f ? a.v_scale / lacc[0] : 0.0f;
    uint16_t* op = (uint16_t*)a.o + ((size_t)b * N + qi) * ((size_t)a.H * D) + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < kDblocks; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = db * 32 + g * 8 + hi * 4;
        u32x2 w;
        w[0] = Bf16Ops::pack2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
        w[1] = Bf16Ops::pack2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
        *(u32x2*)(op + dim) = w;
      }
    if (hi == 0) a.lse[((size_t)b * a.H + h) * N + qi] = (m_run - kOff + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

// ---- host side -------------------------------------------------------------------------
bool aligned(const void* p, size_t n) { return ((uintptr_t)p % n) == 0; }

fa_status check_sizes(int B, int H, int Hkv, int N, int d, int causal, fa_dtype dtype) {
  if (B < 1 || H < 1 || Hkv < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (Hkv > H || H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3)
    return FA_ERR_INVALID_ARG;
  const long long q_elems = (long long)B * N * H * d;
  if (q_elems >= (1LL << 31)) return FA_ERR_INVALID_ARG;
  const long long grid = ((long long)N + kBr - 1) / kBr * H * B;
  if (grid > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // K and V of one batch are addressed through buffer descriptors with 32-bit offsets and
  // a signed 32-bit extent
  const long long kv_batch_bytes = (long long)N * Hkv * d * (dtype == FA_DTYPE_FP8_E4M3 ? 1 : 2);
  if (kv_batch_bytes >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

template <typename Ops, int D, int MASK>
fa_status launch(const FwdArgs& args, hipStream_t stream) {
  fa_env::log_launch("fa_fwd_overlap_kernel", __PRETTY_FUNCTION__, args.total, kThreads);
  hipLaunchKernelGGL((fa_fwd_overlap_kernel<Ops, D, MASK>), dim3(args.total), dim3(kThreads), 0, stream, args);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <int D, int MASK, bool BLOCK = false, bool QK8 = false>
fa_status launch_fp8(const FwdArgs& args, hipStream_t stream) {
  if constexpr (QK8) {
    fa_env::log_launch("fa_fwd_e4m3qk_kernel", __PRETTY_FUNCTION__, args.total, kThreads);
    hipLaunchKernelGGL((fa_fwd_e4m3qk_kernel<D, MASK, BLOCK>), dim3(args.total), dim3(kThreads), 0, stream, args);
  } else {
    fa_env::log_launch("fa_fwd_fp8_kernel", __PRETTY_FUNCTION__, args.total, kThreads);
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, MASK, BLOCK>), dim3(args.total), dim3(kThreads), 0, stream, args);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <typename Ops, int D>
fa_status dispatch_mask(const FwdArgs& args, int mask, hipStream_t stream) {
  switch (mask) {
    case kMaskNone: return launch<Ops, D, kMaskNone>(args, stream);
    case kMaskCausal: return launch<Ops, D, kMaskCausal>(args, stream);
    default: return launch<Ops, D, kMaskBand>(args, stream);
  }
}

template <int D>
fa_status dispatch_fp8(const FwdArgs& args, int mask, hipStream_t stream) {
  switch (mask) {
    case kMaskNone: return launch_fp8<D, kMaskNone>(args, stream);
    case kMaskCausal: return launch_fp8<D, kMaskCausal>(args, stream);
    default: return launch_fp8<D, kMaskBand>(args, stream);
  }
}

// Mask of (causal, window_left, window_right) after normalising the window: a negative or
// too-wide side is unbounded (wl/wr = N), a causal mask bounds the right side at 0. A
// window that bounds nothing is the plain or causal case.
int resolve_mask(int N, int causal, int window_left, int window_right, int* wl, int* wr) {
  *wl = (window_left < 0 || window_left >= N) ? N : window_left;
  *wr = (window_right < 0 || window_right >= N) ? N : window_right;
  if (causal) *wr = 0;
  if (*wl == N && *wr == N) return kMaskNone;
  if (*wl == N && *wr == 0) return kMaskCausal;
  return kMaskBand;
}

fa_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int Hkv, int N, int d, int causal, int window_left, int window_right,
                   float scale, fa_dtype dtype, const float* descale_qkv, void* stream);

void fill_common(FwdArgs& args, const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int H, int Hkv, int N) {
  args.q = q;
  args.k = k;
  args.v = v;
  args.o = o;
  args.lse = lse;
  args.B = B;
  args.H = H;
  args.Hkv = Hkv;
  args.N = N;
  args.group = H / Hkv;
  args.num_qtiles = (N + kBr - 1) / kBr;
  args.total = args.num_qtiles * H * B;
  args.q_scales = args.k_scales = args.v_scales = nullptr;
  args.nb = (N + FA_FP8_BLOCK_ROWS - 1) / FA_FP8_BLOCK_ROWS;
  args.block_mask = nullptr;
  args.mask_heads = 1;
  args.nblk = (N + kSparseBlock - 1) / kSparseBlock;
}

fa_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int Hkv, int N, int d, int causal, int window_left, int window_right,
                   float scale, fa_dtype dtype, const float* descale_qkv, void* stream) {
  fa_status st = check_sizes(B, H, Hkv, N, d, causal, dtype);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if (dtype == FA_DTYPE_FP8_E4M3) {
    if (!descale_qkv) return FA_ERR_INVALID_ARG;
    for (int i = 0; i < 3; ++i)
      if (!std::isfinite(descale_qkv[i]) || !(descale_qkv[i] > 0.0f)) return FA_ERR_INVALID_ARG;
  } else if (descale_qkv) {
    return FA_ERR_INVALID_ARG;
  }
  FwdArgs args;
  fill_common(args, q, k, v, o, lse, B, H, Hkv, N);
  args.c = (float)((double)scale * 1.4426950408889634);
  args.v_scale = 1.0f;
  const int mask = resolve_mask(N, causal, window_left, window_right, &args.wl, &args.wr);
  if (dtype == FA_DTYPE_FP8_E4M3) {
    args.c = (float)((double)scale * descale_qkv[0] * descale_qkv[1] * 1.4426950408889634);
    args.v_scale = descale_qkv[2];
  }
  hipStream_t s = (hipStream_t)stream;
  switch (dtype) {
    case FA_DTYPE_BF16:
      return d == 128 ? dispatch_mask<Bf16Ops, 128>(args, mask, s) : dispatch_mask<Bf16Ops, 64>(args, mask, s);
    case FA_DTYPE_F16:
      return d == 128 ? dispatch_mask<F16Ops, 128>(args, mask, s) : dispatch_mask<F16Ops, 64>(args, mask, s);
    case FA_DTYPE_FP8_E4M3:
      return d == 128 ? dispatch_fp8<128>(args, mask, s) : dispatch_fp8<64>(args, mask, s);
    default: return FA_ERR_UNSUPPORTED;
  }
}

template <typename Ops, int D>
fa_status launch_block_sparse(const FwdArgs& args, int causal, hipStream_t stream) {
  return causal ? launch<Ops, D, kMaskBlockCausal>(args, stream) : launch<Ops, D, kMaskBlock>(args, stream);
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int Hkv, int N, int d, int causal, float scale, fa_dtype dtype,
                 const float* descale_qkv, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, causal, -1, -1, scale, dtype, descale_qkv, stream);
}

fa_status fa_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int Hkv, int N, int d, int causal, int window_left,
                       int window_right, float scale, fa_dtype dtype, const float* descale_qkv,
                       void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, causal, window_left, window_right, scale, dtype,
                  descale_qkv, stream);
}

fa_status fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                              int H, int Hkv, int N, int d, int causal, const unsigned char* block_mask,
                              int mask_heads, float scale, fa_dtype dtype, void* stream) {
  fa_status st = check_sizes(B, H, Hkv, N, d, causal, dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_DTYPE_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o || !lse || !block_mask) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID_ARG;
  if (mask_heads != 1 && mask_heads != H) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if ((N + kSparseBlock - 1) / kSparseBlock > kMaxSparseBlocks) return FA_ERR_UNSUPPORTED;
  FwdArgs args;
  fill_common(args, q, k, v, o, lse, B, H, Hkv, N);
  args.c = (float)((double)scale * 1.4426950408889634);
  args.v_scale = 1.0f;
  args.wl = args.wr = N;
  args.block_mask = block_mask;
  args.mask_heads = mask_heads;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == FA_DTYPE_BF16)
    return d == 128 ? launch_block_sparse<Bf16Ops, 128>(args, causal, s) : launch_block_sparse<Bf16Ops, 64>(args, causal, s);
  return d == 128 ? launch_block_sparse<F16Ops, 128>(args, causal, s) : launch_block_sparse<F16Ops, 64>(args, causal, s);
}

fa_status fa_fwd_fp8_block(const void* q, const void* k, const void* v, const unsigned char* q_scales,
                           const unsigned char* k_scales, const unsigned char* v_scales, void* o,
                           float* lse, int B, int H, int Hkv, int N, int d, int causal, float scale,
                           int qk_e4m3, void* stream) {
  fa_status st = check_sizes(B, H, Hkv, N, d, causal, FA_DTYPE_FP8_E4M3);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !lse || !q_scales || !k_scales || !v_scales) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if (qk_e4m3 != 0 && qk_e4m3 != 1) return FA_ERR_INVALID_ARG;
  if ((N + kBc - 1) / kBc > kMaxScaleTiles) return FA_ERR_UNSUPPORTED;
  if (fa_env::forced_fp8_block_qk() >= 0) qk_e4m3 = fa_env::forced_fp8_block_qk();
  FwdArgs args;
  fill_common(args, q, k, v, o, lse, B, H, Hkv, N);
  args.c = (float)((double)scale * 1.4426950408889634);
  args.v_scale = 1.0f;       // the V block scales are applied inside the P.V MFMA
  args.wl = args.wr = N;
  args.q_scales = q_scales;
  args.k_scales = k_scales;
  args.v_scales = v_scales;
  hipStream_t s = (hipStream_t)stream;
  if (qk_e4m3) {
    if (d == 128) return causal ? launch_fp8<128, kMaskCausal, true, true>(args, s) : launch_fp8<128, kMaskNone, true, true>(args, s);
    return causal ? launch_fp8<64, kMaskCausal, true, true>(args, s) : launch_fp8<64, kMaskNone, true, true>(args, s);
  }
  if (d == 128) return causal ? launch_fp8<128, kMaskCausal, true>(args, s) : launch_fp8<128, kMaskNone, true>(args, s);
  return causal ? launch_fp8<64, kMaskCausal, true>(args, s) : launch_fp8<64, kMaskNone, true>(args, s);
}

fa_status fa_fwd_query(int B, int H, int Hkv, int N, int d, int causal, fa_dtype dtype,
                       size_t* q_bytes, size_t* kv_bytes, size_t* o_bytes, size_t* lse_bytes,
                       size_t* workspace_bytes) {
  fa_status st = check_sizes(B, H, Hkv, N, d, causal, dtype);
  if (st != FA_OK) return st;
  const size_t in_size = dtype == FA_DTYPE_FP8_E4M3 ? 1 : 2;
  if (q_bytes) *q_bytes = (size_t)B * N * H * d * in_size;
  if (kv_bytes) *kv_bytes = (size_t)B * N * Hkv * d * in_size;
  if (o_bytes) *o_bytes = (size_t)B * N * H * d * 2;
  if (lse_bytes) *lse_bytes = (size_t)B * H * N * sizeof(float);
  if (workspace_bytes) *workspace_bytes = 0;
  return FA_OK;
}

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported configuration";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: the request needs more than the library's static scratch";
  }
  return "unknown fa_status";
}

int fa_version(void) { return 10300; }

}  // extern "C"
