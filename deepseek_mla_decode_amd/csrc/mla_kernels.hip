// mla_kernels.hip -- gfx950 (CDNA4) kernels of the MLA decode library.
//
// Three kernels:
//   * plan_kernel    one workgroup; turns cache_seqlens into the split plan.
//   * split_kernel   one workgroup per (work item, head group of 128 heads);
//                    streams the work item's KV rows through LDS and runs the
//                    base-2 online softmax with both products on MFMA.
//   * combine_kernel merges the per-split partials of sequences with s_b > 1.
//
// What is computed follows the TileLang MLA guide ("用 TileLang 编写高性能
// DeepSeek MLA 内核"): "Split Kernel" (score tile = q_nope·latentᵀ + q_pe·ropeᵀ
// accumulated together; running max / rescale / running sum in base 2 with
// softmax_scale·log2(e) folded into one multiply-add; P rounded to the input
// type before the P·V product; the partial is normalised and its base-2 lse is
// log2(sum) + max), "Combine Kernel" (anchor at the largest partial lse, total
// = log2 Σ 2^(lse_k - anchor) + anchor, weights 2^(lse_k - total)), and the
// FlashMLA analysis ("DeepSeek开源周第一天：FlashMLA 深度分析"), "Softmax 计算
//优化" (a row whose max is -inf uses 0 as the max so that no -inf - -inf
// appears).  The CDNA4 design (tile shapes, operand placement, LDS layout,
// lazy rescale) is this library's own; see the comments at each step.
//
// split_kernel in brief (256 threads = 4 waves, one wave per SIMD):
//   * wave w owns query heads [32w, 32w + 32) of the group; lane l serves head
//     l % 32 and half g = l / 32 of the contraction slots of every MFMA.
//   * Scores are formed transposed, Sᵀ[n][h] = K[n][:]·Q[h][:], with
//     v_mfma_f32_32x32x16: A = 32 cache rows × 16 dims read from LDS, B = the
//     wave's Q slice held in 144 VGPRs for the whole work item.  Each lane then
//     holds 16 scores of ONE head, so max/sum need a single cross-lane step
//     (lane l ^ 32) and P is already laid out as the B operand of P·V.
//   * Output is also transposed, Oᵀ[v][h] += Vᵀ[v][n]·Pᵀ[n][h]: 16 MFMA tiles
//     of 32 value columns, accumulator 32 heads × 512 fp32 = 256 AGPRs; every
//     value a lane holds belongs to its own head, so rescaling is lane-local.
//     The Vᵀ operand is read straight from the row-major tile with gfx950's
//     transposing LDS read (ds_read_b64_tr_b16): no second copy of the tile.
//   * Cache rows go HBM -> LDS with global_load_lds_dwordx4 (no VGPRs): one
//     instruction moves one 1 KiB latent row (or eight 128-byte RoPE rows).
//     A ring of 4 tiles of 32 rows (36 KiB each) keeps 3 tiles in flight
//     while one is computed; one barrier per tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_rule.h"
#include "mla_kernels.h"

namespace mla {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileRows = 32;                 // cache rows per LDS tile
constexpr int kThreads = 256;                 // 4 waves
constexpr float kLn2 = 0.69314718055994530942f;

// ---------------------------------------------------------------------------
// dtype helpers
// ---------------------------------------------------------------------------

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == MLA_DTYPE_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// MFMAs written as inline asm.  The constraint letter pins the accumulator:
// "v" for the per-tile score tile, "a" for the P·V accumulator, which owns all
// 256 AGPRs.  (Left to itself the register allocator puts the score tile in
// AGPRs and pushes part of the P·V accumulator out, and then spills.)  The
// asm statements also fix the issue order, so the LDS reads below are
// software-pipelined by hand: an operand is read three MFMAs ahead of use.
// Hazards the compiler cannot see through asm are covered by explicit
// s_nop: VALU-written operands before the first MFMA of a group, and MFMA
// results before VALU reads them.
template <int DT, bool FIRST>
__device__ __forceinline__ void mfma_v(f32x16& c, u32x4 a, u32x4 b) {
  if constexpr (DT == MLA_DTYPE_F16) {
    if constexpr (FIRST) asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    else asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  } else {
    if constexpr (FIRST) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  }
}

template <int DT>
__device__ __forceinline__ void mfma_a(f32x16& c, u32x4 a, u32x4 b) {
  if constexpr (DT == MLA_DTYPE_F16) asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Wait states between an MFMA writing a register and a VALU instruction
// reading it (>= 18 for the 16-pass 32x32 shapes), and between VALU writes
// and an MFMA reading them.  The registers concerned are asm operands, so no
// read (or write) of them can be scheduled across the s_nop block.
__device__ __forceinline__ void nops_after_mfma(f32x16& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(c));
}
__device__ __forceinline__ void nops_after_mfma(f32x16 (&acc)[16]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory");
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("" : "+a"(acc[i]));
}
template <int DT>
__device__ __forceinline__ void nops_before_mfma(u32x4 (&x)[2], u32x4 (&y)[2]) {
  if constexpr (DT == MLA_DTYPE_F16) asm volatile("s_nop 4" : "+v"(x[0]), "+v"(x[1]));
  else asm volatile("s_nop 4" : "+v"(x[0]), "+v"(x[1]), "+v"(y[0]), "+v"(y[1]));
}

// Reductions across the two halves of a wave (lane l with lane l ^ 32) through
// v_permlane32_swap, a VALU op: it exchanges the upper half of its first
// register with the lower half of its second, so afterwards one register holds
// this lane's value and the other its partner's, and max / sum of the pair is
// the same in both halves.  Written as asm with two distinct registers: the
// builtin, given the same value twice, is folded as if both results were equal.
// The leading s_nop covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float halves_max(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float halves_sum(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return a + b;
}

// Round-to-nearest-even fp32 -> 16-bit storage of the input type.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == MLA_DTYPE_F16) {
    _Float16 a = (_Float16)lo, b = (_Float16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  } else {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// ---------------------------------------------------------------------------
// LDS tile layout
// ---------------------------------------------------------------------------
// One tile = 32 cache rows: a latent region [32][1024 B] followed by a RoPE
// region [32][128 B].  gfx950 serves LDS reads 256 bytes (64 banks) at a time:
// 16 lanes of a 16-byte read, 32 lanes of an 8-byte read.  Chunks are XOR
// swizzled so that both operand reads are conflict-free:
//   latent: 16-byte chunk c of row n at slot c ^ swz_lat(n), swz_lat(n) =
//     4(n % 4) + (n / 4) % 4, distinct over any 16 consecutive rows (score
//     operand: 16 rows of one chunk) and mapping 4 consecutive rows onto the
//     four 4-chunk quarters of a 256-byte line (transposing value read: 4 rows
//     x 4 chunks);
//   RoPE (128-byte rows, two per line): chunk c of row n at slot
//     c ^ ((n / 2) % 8).
constexpr int kLatBytes = kTileRows * 1024;        // 32768
constexpr int kRopeBytes = kTileRows * 128;        // 4096
constexpr int kTileBytes = kLatBytes + kRopeBytes; // 36864
constexpr int kStages = 3;                         // tiles resident in LDS
constexpr int kQRegSteps = 24;                     // k-steps of Q held in VGPRs; the rest in LDS
constexpr int kQLdsBytes = (36 - kQRegSteps) * 4 * 1024;
constexpr int kLoadsPerTile = 9;                   // DMA instructions per wave per tile

__device__ __forceinline__ int swz_lat(int n) { return ((n & 3) << 2) | ((n >> 2) & 3); }
__device__ __forceinline__ int swz_rope(int n) { return (n >> 1) & 7; }

typedef short s16x4 __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) char lds_char;
typedef const __attribute__((address_space(1))) void* gptr_t;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ u32x4 lds_get16(const lds_char* base, int byte_off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base + byte_off);
}

// Two transposing reads give the 8 contraction values of one A operand.
__device__ __forceinline__ u32x4 lds_get_tr(const lds_char* base, int off0, int off1) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + off0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + off1));
  u32x2 a2 = __builtin_bit_cast(u32x2, a), b2 = __builtin_bit_cast(u32x2, b);
  return u32x4{a2.x, a2.y, b2.x, b2.y};
}

// ---------------------------------------------------------------------------
// Split kernel
// ---------------------------------------------------------------------------

// Start of the latent (which == 0) or RoPE (which == 1) part of cache row r;
// `sel` is the sequence (contiguous) or the physical page (paged).
template <bool PAGED>
__device__ __forceinline__ const uint16_t* row_ptr(const SplitParams& p, int64_t sel, int r, int which) {
  const int rr = PAGED ? (r % p.page_size) : r;
  if (which == 0) return p.kv + sel * p.kv_sb + (int64_t)rr * p.kv_sr;
  return p.kpe + sel * p.kpe_sb + (int64_t)rr * p.kpe_sr;
}

// Issue this wave's 9 direct-to-LDS loads of tile rows [tile_base, +32):
// latent rows 8w..8w+7 and the RoPE parts of the same rows.  Rows at or past
// r1 are redirected to row r1 - 1 (always valid); their scores are masked.
// One direct-to-LDS load: 64 lanes x 16 bytes from base + voff (per lane) into
// the 1 KiB of LDS at lds_addr (lane l -> lds_addr + 16 l).  Issued through
// inline asm so that the compiler does not add its own conservative waits for
// the LDS write before every LDS read; the vector-memory counter is managed
// explicitly by the caller (wait_vmcnt).
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(voff), "s"(base)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const lds_char* p) { return (uint32_t)(uintptr_t)p; }

template <bool PAGED>
__device__ __forceinline__ void load_tile(const SplitParams& p, int b, int tile_base, int r1, int wave, int lane,
                                          lds_char* tile) {
  // `wave`, `tile_base`, `r1` are wave-uniform: row and page arithmetic stays
  // scalar; only the swizzled 16-byte lane offset is per lane.
  int64_t sel;
  if constexpr (PAGED) {
    const int pg = p.block_table[(int64_t)b * p.bt_stride + tile_base / p.page_size];
    sel = pg < 0 ? 0 : (pg >= p.num_pages ? p.num_pages - 1 : pg);
  } else {
    sel = b;
  }
  const int last = r1 - 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = 8 * wave + i;
    int r = tile_base + n;
    r = r < last ? r : last;
    dma16(row_ptr<PAGED>(p, sel, r, 0), 16u * (uint32_t)(lane ^ swz_lat(n)), lds_u32(tile + n * 1024));
  }
  // RoPE: lane l carries row 8w + l/8, slot l % 8 (holding chunk slot ^ swz_rope(row)).
  // The eight rows are not contiguous in memory, so the lane offset is taken
  // from the first row of the group.
  const int n0 = 8 * wave;
  const int n = n0 + (lane >> 3);
  int r = tile_base + n;
  r = r < last ? r : last;
  int rf = tile_base + n0;
  rf = rf < last ? rf : last;
  const char* first = reinterpret_cast<const char*>(row_ptr<PAGED>(p, sel, rf, 1));
  const char* mine = reinterpret_cast<const char*>(row_ptr<PAGED>(p, sel, r, 1));
  dma16(first, (uint32_t)(mine - first) + 16u * (uint32_t)((lane & 7) ^ swz_rope(n)),
        lds_u32(tile + kLatBytes + n0 * 128));
}

// Q slice of this lane's head: k-step s (dims 16s .. 16s+15, this lane's half
// g) is the B operand of the score MFMA.  The first kQRegSteps k-steps stay in
// VGPRs; the rest go to LDS at [step][wave][lane] 16-byte slots.
__device__ __forceinline__ void load_q(const SplitParams& p, int b, int h, bool head_ok, int wave, int lane,
                                       lds_char* qlds, u32x4 (&qreg)[kQRegSteps]) {
  const int g = lane >> 5;
  const uint16_t* qn = p.q_nope + (int64_t)b * p.q_nope_sb + (int64_t)h * p.q_nope_sh + 8 * g;
  const uint16_t* qp = p.q_pe + (int64_t)b * p.q_pe_sb + (int64_t)h * p.q_pe_sh + 8 * g;
#pragma unroll
  for (int s = 0; s < 36; ++s) {
    u32x4 v = s < 32 ? ld16(qn + 16 * s) : ld16(qp + 16 * (s - 32));
    v = head_ok ? v : u32x4{0u, 0u, 0u, 0u};
    if (s < kQRegSteps) qreg[s < kQRegSteps ? s : 0] = v;
    else *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(qlds + ((s - kQRegSteps) * 4 + wave) * 1024 + 16 * lane) = v;
  }
}

// REDO = false: the main pass.  REDO = true: the second launch, which only
// reruns work items whose main pass flagged an overflow (see below).
template <int DT, bool PAGED, bool REDO>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void split_kernel(SplitParams p) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[kStages * kTileBytes + kQLdsBytes];
  __shared__ int overflow;
  lds_char* lds = (lds_char*)lds_raw;
  lds_char* qlds = lds + kStages * kTileBytes;

  const int wi = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hl = lane & 31;
  const int g = lane >> 5;

  // ---- work item (uniform) -------------------------------------------------
  int b, r0, r1, s_b;
  if (p.num_split > 0) {
    b = wi / p.num_split;
    const int k = wi - b * p.num_split;
    split_range(clamp_len(p.seqlens[b], p.row_cap), p.num_split, k, &r0, &r1);
    s_b = p.num_split;
  } else {
    if (wi >= p.split_offset[p.batch]) return;
    b = p.work[4 * wi + 0];
    r0 = p.work[4 * wi + 2];
    r1 = p.work[4 * wi + 3];
    s_b = p.split_offset[b + 1] - p.split_offset[b];
  }
  if (REDO && p.redo[wi] == 0) return;
  b = __builtin_amdgcn_readfirstlane(b);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  r1 = __builtin_amdgcn_readfirstlane(r1);
  s_b = __builtin_amdgcn_readfirstlane(s_b);
  const int n_tiles = (r1 - r0 + kTileRows - 1) / kTileRows;

  // Heads of this wave.  Lanes past the last head compute with a zero query
  // and write nothing.
  const int h0 = blockIdx.y * kHeadsPerGroup + wave * 32;
  const bool head_ok = h0 + hl < p.heads;
  const int h = head_ok ? h0 + hl : p.heads - 1;

  u32x4 qreg[kQRegSteps];
  load_q(p, b, h, head_ok, wave, lane, qlds, qreg);
  if (threadIdx.x == 0) overflow = 0;   // published by the first barrier

  // Per-lane LDS byte offsets inside a tile.
  //   Score operand, k-step s < 32 (row hl, chunk 2s+g):
  //     klat + 256 (s / 8) + 16 ((2 (s % 8)) ^ kx), kx = g ^ swz_lat(hl).
  //   RoPE k-step s >= 32 (chunk 2(s-32)+g): krope + 16 ((2(s-32) + g) ^ swz_rope(hl)).
  //   Transposing value read for column block vb, k-step kt, half r:
  //     (vofs[r] ^ 64 (vb % 4)) + 256 (vb / 4) + 16384 kt + 8192 r.
  const int klat = hl * 1024;
  const int kx = g ^ swz_lat(hl);
  const int krope = kLatBytes + hl * 128;
  const int kxr = swz_rope(hl);
  int vofs[2];
  {
    const int i = lane & 15, G = lane >> 4;
    const int y = 2 * (G & 1) + ((i >> 1) & 1);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int z = (2 * r + (G >> 1)) & 3;
      vofs[r] = 4096 * (G >> 1) + 1024 * (i >> 2) + 64 * (i >> 2) + 16 * (y ^ z) + 8 * (i & 1);
    }
  }
  const int qofs = wave * 1024 + 16 * lane;

  // The exponentials use a reference max `m` that does not change during the
  // pass over the tiles (changing it would mean rescaling the accumulator,
  // which must never leave the AGPRs).  The main pass takes m from the first
  // tile, so P = 2^(x - m) may exceed 1; that is exact while P stays inside the
  // range of the P·V operand type.  If some tile's max passes m by more than
  // kOverflowMargin, the main pass writes no output: it flags the work item
  // and stores the exact max (`mx`, the max over all tiles); the REDO launch
  // then recomputes the work item with m = mx, where P <= 1.
  constexpr float kOverflowMargin = DT == MLA_DTYPE_F16 ? 15.0f : 64.0f;
  f32x16 acc[16];
#pragma unroll
  for (int vb = 0; vb < 16; ++vb) acc[vb] = f32x16{};
  float m = REDO ? p.part_lse[(int64_t)wi * p.heads + h] : -__builtin_inff();
  float mx = -__builtin_inff();   // running max of all tiles seen
  float lsum = 0.f;               // this lane's share of the sum of P

  // Prologue: up to three tiles in flight.
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (i < n_tiles) load_tile<PAGED>(p, b, r0 + i * kTileRows, r1, wave, lane, lds + i * kTileBytes);

  for (int t = 0; t < n_tiles; ++t) {
    const int tile_base = r0 + t * kTileRows;
    // Tile t has landed once only the loads of the tiles after it that are
    // already issued (at most kStages - 2 of them) are pending.
    static_assert(kStages == 3, "wait counts below assume a three-tile ring");
    if (t + 1 < n_tiles) wait_vmcnt<kLoadsPerTile>();
    else wait_vmcnt<0>();
    // Barrier without a memory fence: the only cross-wave data are the DMA
    // tiles, whose arrival each wave has just waited for.  The "memory"
    // clobber keeps LDS reads from moving above it.
    asm volatile("s_barrier" ::: "memory");
    if (t + kStages - 1 < n_tiles)
      load_tile<PAGED>(p, b, tile_base + (kStages - 1) * kTileRows, r1, wave, lane,
                       lds + ((t + kStages - 1) % kStages) * kTileBytes);

    const lds_char* tile = lds + (t % kStages) * kTileBytes;
    // -- scores: Sᵀ[n][h], n = 8(e/4) + 4g + (e%4) for accumulator element e.
    //    K operand of k-step s: row hl, chunk 2s+g (RoPE chunks after 32);
    //    Q operand: VGPRs for s < kQRegSteps, else this wave's LDS slots.
    f32x16 sacc;
    {
      u32x4 kb[5], qb[5];
      auto kaddr = [&](int s) -> int {
        return s < 32 ? klat + 256 * (s >> 3) + 16 * ((2 * (s & 7)) ^ kx) : krope + 16 * ((2 * (s - 32) + g) ^ kxr);
      };
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        kb[s] = lds_get16(tile, kaddr(s));
        if (s >= kQRegSteps) qb[s] = lds_get16(qlds, qofs + (s - kQRegSteps) * 4096);
      }
#pragma unroll
      for (int s = 0; s < 36; ++s) {
        if (s + 3 < 36) {
          kb[(s + 3) % 5] = lds_get16(tile, kaddr(s + 3));
          if (s + 3 >= kQRegSteps) qb[(s + 3) % 5] = lds_get16(qlds, qofs + (s + 3 - kQRegSteps) * 4096);
        }
        const u32x4 q = s < kQRegSteps ? qreg[s < kQRegSteps ? s : 0] : qb[s % 5];
        if (s == 0) mfma_v<DT, true>(sacc, kb[0], q);
        else mfma_v<DT, false>(sacc, kb[s % 5], q);
      }
      nops_after_mfma(sacc);
    }

    float x[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = sacc[e] * p.scale_log2;
    if (tile_base + kTileRows > r1) {   // last tile: mask rows at or past r1
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int n = 8 * (e >> 2) + 4 * g + (e & 3);
        if (tile_base + n >= r1) x[e] = -__builtin_inff();
      }
    }
    float tmax = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, x[e]);
    tmax = halves_max(tmax);
    mx = fmaxf(mx, tmax);
    if (!REDO) {
      if (t == 0) m = tmax;
      else if (__any(tmax > m + kOverflowMargin) && lane == 0) overflow = 1;
    }
    const float mu = (m == -__builtin_inff()) ? 0.f : m;

    // -- P = 2^(x - m) as the B operand of P·V.  fp16: P rounded to fp16.
    //    bf16: P = hi + lo, both bf16, so the product keeps ~16 bits of P.
    float pv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pv[e] = __builtin_amdgcn_exp2f(x[e] - mu);
      lsum += pv[e];
    }
    u32x4 pk[2], pl[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      uint32_t w[4], wl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = pv[8 * kt + 2 * j], cc = pv[8 * kt + 2 * j + 1];
        w[j] = pack2<DT>(a, cc);
        if constexpr (DT == MLA_DTYPE_BF16) {
          const float ah = __builtin_bit_cast(float, w[j] << 16);
          const float ch = __builtin_bit_cast(float, w[j] & 0xFFFF0000u);
          wl[j] = pack2<DT>(a - ah, cc - ch);
        }
      }
      pk[kt] = u32x4{w[0], w[1], w[2], w[3]};
      if constexpr (DT == MLA_DTYPE_BF16) pl[kt] = u32x4{wl[0], wl[1], wl[2], wl[3]};
    }

    // -- Oᵀ[v][h] += Vᵀ[v][n] Pᵀ[n][h] over 16 blocks of 32 value columns.
    //    Contraction slot (g, j) of k-step kt is row 16kt + 8(j/4) + 4g + (j%4),
    //    the layout in which the score MFMA leaves P.  Operand i = 2vb + kt is
    //    read with two transposing loads, three operands ahead.
    {
      // operand i = 2 vb + kt
      auto vaddr = [&](int i, int r) -> int {
        const int vb = i >> 1, kt = i & 1;
        return (vofs[r] ^ (64 * (vb & 3))) + 256 * (vb >> 2) + 16384 * kt + 8192 * r;
      };
      u32x4 vbuf[5];
#pragma unroll
      for (int i = 0; i < 3; ++i) vbuf[i] = lds_get_tr(tile, vaddr(i, 0), vaddr(i, 1));
      nops_before_mfma<DT>(pk, pl);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i + 3 < 32) vbuf[(i + 3) % 5] = lds_get_tr(tile, vaddr(i + 3, 0), vaddr(i + 3, 1));
        mfma_a<DT>(acc[i >> 1], vbuf[i % 5], pk[i & 1]);
        if constexpr (DT == MLA_DTYPE_BF16) mfma_a<DT>(acc[i >> 1], vbuf[i % 5], pl[i & 1]);
      }
    }

  }
  nops_after_mfma(acc);
  if (!REDO) {
    // Every wave's overflow flag write is visible after this barrier.
    __syncthreads();
    if (overflow) {
      if (threadIdx.x == 0) p.redo[wi] = 1;
      if (head_ok && g == 0) p.part_lse[(int64_t)wi * p.heads + h] = mx;
      return;
    }
    if (threadIdx.x == 0) p.redo[wi] = 0;
  }

  // ---- epilogue: normalise; write final output or the split partial --------
  const float ltot = halves_sum(lsum);
  const bool nonempty = ltot > 0.f;
  const float inv = nonempty ? 1.f / ltot : 0.f;
  const float lse2 = nonempty ? __log2f(ltot) + m : -__builtin_inff();
  if (!head_ok) return;
  if (s_b == 1) {
    uint16_t* o = p.out + (int64_t)b * p.out_sb + (int64_t)h * p.out_sh;
#pragma unroll
    for (int vb = 0; vb < 16; ++vb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int v = 32 * vb + 8 * q + 4 * g;
        u32x2 w;
        w.x = pack2<DT>(acc[vb][4 * q + 0] * inv, acc[vb][4 * q + 1] * inv);
        w.y = pack2<DT>(acc[vb][4 * q + 2] * inv, acc[vb][4 * q + 3] * inv);
        *reinterpret_cast<u32x2*>(o + v) = w;
      }
    }
    if (g == 0) p.lse[(int64_t)b * p.heads + h] = nonempty ? lse2 * kLn2 : -__builtin_inff();
  } else {
    float* o = p.part_o + ((int64_t)wi * p.heads + h) * 512;
#pragma unroll
    for (int vb = 0; vb < 16; ++vb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int v = 32 * vb + 8 * q + 4 * g;
        f32x4 w = {acc[vb][4 * q + 0] * inv, acc[vb][4 * q + 1] * inv, acc[vb][4 * q + 2] * inv,
                   acc[vb][4 * q + 3] * inv};
        *reinterpret_cast<f32x4*>(o + v) = w;
      }
    }
    if (g == 0) p.part_lse[(int64_t)wi * p.heads + h] = lse2;
  }
}

// ---------------------------------------------------------------------------
// Combine kernel: grid (ceil(H / 4), B), one wave per head, 8 values per lane.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int DT>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int b = blockIdx.y;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (h >= p.heads) return;
  int s, base;
  if (p.num_split > 0) {
    s = p.num_split;
    base = b * p.num_split;
  } else {
    base = p.split_offset[b];
    s = p.split_offset[b + 1] - base;
  }
  if (s <= 1) return;

  const float* L = p.part_lse + (int64_t)base * p.heads + h;
  float mx = -__builtin_inff();
  for (int k = lane; k < s; k += 64) mx = fmaxf(mx, L[(int64_t)k * p.heads]);
  mx = wave_max(mx);

  uint16_t* o = p.out + (int64_t)b * p.out_sb + (int64_t)h * p.out_sh + 8 * lane;
  if (mx == -__builtin_inff()) {
    *reinterpret_cast<u32x4*>(o) = u32x4{0u, 0u, 0u, 0u};
    if (lane == 0) p.lse[(int64_t)b * p.heads + h] = -__builtin_inff();
    return;
  }
  float se = 0.f;
  for (int k = lane; k < s; k += 64) se += __builtin_amdgcn_exp2f(L[(int64_t)k * p.heads] - mx);
  se = wave_sum(se);
  const float total = __log2f(se) + mx;

  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  const float* O = p.part_o + ((int64_t)base * p.heads + h) * 512 + 8 * lane;
  for (int k = 0; k < s; ++k) {
    const float w = __builtin_amdgcn_exp2f(L[(int64_t)k * p.heads] - total);
    const f32x4* src = reinterpret_cast<const f32x4*>(O + (int64_t)k * p.heads * 512);
    a0 += w * src[0];
    a1 += w * src[1];
  }
  u32x4 r;
  r.x = pack2<DT>(a0.x, a0.y);
  r.y = pack2<DT>(a0.z, a0.w);
  r.z = pack2<DT>(a1.x, a1.y);
  r.w = pack2<DT>(a1.z, a1.w);
  *reinterpret_cast<u32x4*>(o) = r;
  if (lane == 0) p.lse[(int64_t)b * p.heads + h] = total * kLn2;
}

// ---------------------------------------------------------------------------
// Planner kernel: one workgroup of 1024 threads.
// ---------------------------------------------------------------------------

constexpr int kPlanThreads = 1024;

__device__ int block_sum(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int tot = 0;
  for (int i = 0; i < kPlanThreads / 64; ++i) tot += red[i];
  return tot;
}

__device__ int block_max(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int m = 0;
  for (int i = 0; i < kPlanThreads / 64; ++i) m = max(m, red[i]);
  return m;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanParams p) {
  __shared__ int red[kPlanThreads / 64];
  __shared__ int scan[kPlanThreads];
  const int B = p.batch;
  const int tid = threadIdx.x;

  // Budget t: forced mode uses s_b = num_split; planner mode searches the
  // smallest t whose split total fits the cap.
  int t = 1;
  if (p.num_split == 0) {
    int mx = 0;
    for (int b = tid; b < B; b += kPlanThreads) mx = max(mx, num_blocks(clamp_len(p.seqlens[b], p.row_cap)));
    mx = block_max(mx, red);
    const int cap = planner_cap(B, p.heads, p.num_cus);
    int lo = 1, hi = mx > 1 ? mx : 1;
    while (lo < hi) {
      const int mid = lo + (hi - lo) / 2;
      int cnt = 0;
      for (int b = tid; b < B; b += kPlanThreads)
        cnt += splits_for_budget(num_blocks(clamp_len(p.seqlens[b], p.row_cap)), mid);
      cnt = block_sum(cnt, red);
      if (cnt <= cap) hi = mid; else lo = mid + 1;
    }
    t = lo;
  }

  // Contiguous chunk of sequences per thread; exclusive scan of chunk totals.
  const int per = (B + kPlanThreads - 1) / kPlanThreads;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int mine = 0;
  for (int b = b0; b < b1; ++b)
    mine += p.num_split > 0 ? p.num_split : splits_for_budget(num_blocks(clamp_len(p.seqlens[b], p.row_cap)), t);
  __syncthreads();
  scan[tid] = mine;
  __syncthreads();
  for (int o = 1; o < kPlanThreads; o <<= 1) {
    const int v = tid >= o ? scan[tid - o] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int off = scan[tid] - mine;
  for (int b = b0; b < b1; ++b) {
    const int L = clamp_len(p.seqlens[b], p.row_cap);
    const int s = p.num_split > 0 ? p.num_split : splits_for_budget(num_blocks(L), t);
    p.num_splits[b] = s;
    p.split_offset[b] = off;
    for (int k = 0; k < s; ++k) {
      int r0, r1;
      split_range(L, s, k, &r0, &r1);
      int* w = p.work + 4 * (off + k);
      w[0] = b;
      w[1] = k;
      w[2] = r0;
      w[3] = r1;
    }
    off += s;
  }
  if (tid == kPlanThreads - 1) p.split_offset[B] = scan[kPlanThreads - 1];
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

hipError_t launch_plan(const PlanParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

template <bool REDO>
static void launch_split_t(const SplitParams& p, int dtype, bool paged, dim3 grid, hipStream_t stream) {
  const dim3 block(kThreads);
  if (dtype == MLA_DTYPE_F16) {
    if (paged) hipLaunchKernelGGL((split_kernel<MLA_DTYPE_F16, true, REDO>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((split_kernel<MLA_DTYPE_F16, false, REDO>), grid, block, 0, stream, p);
  } else {
    if (paged) hipLaunchKernelGGL((split_kernel<MLA_DTYPE_BF16, true, REDO>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((split_kernel<MLA_DTYPE_BF16, false, REDO>), grid, block, 0, stream, p);
  }
}

hipError_t launch_split(const SplitParams& p, int dtype, bool paged, int grid_x, int grid_y, bool redo,
                        hipStream_t stream) {
  const dim3 grid(grid_x, grid_y);
  if (redo) launch_split_t<true>(p, dtype, paged, grid, stream);
  else launch_split_t<false>(p, dtype, paged, grid, stream);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int dtype, int batch, hipStream_t stream) {
  const dim3 grid((p.heads + 3) / 4, batch), block(256);
  if (dtype == MLA_DTYPE_F16) hipLaunchKernelGGL(combine_kernel<MLA_DTYPE_F16>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(combine_kernel<MLA_DTYPE_BF16>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
