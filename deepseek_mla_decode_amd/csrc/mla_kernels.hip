// mla_kernels.hip -- gfx950 (CDNA4) kernels of the MLA decode library.
//
// Kernels:
//   * plan_kernel    one workgroup; turns cache_seqlens into the split plan
//                    (the stand-alone planner entry point; decode itself plans
//                    inside split_kernel, every wave for its own work item, or
//                    reads its item from a plan made beforehand: the GIVEN
//                    instances).
//   * split_kernel   one workgroup per (work item, head group of 128 heads);
//                    streams the work item's KV rows through LDS and runs the
//                    base-2 online softmax with both products on MFMA.  With
//                    an FP8 (E4M3) cache the rows arrive as bytes and each
//                    wave widens its share of a tile to 16 bits in LDS.
//   * combine_heads_kernel / combine_splitk_kernel merge the per-split
//                    partials of sequences with s_b > 1: one wave per head for
//                    few splits, four waves over the splits of a head for many.
//   * check_block_table_kernel  counts block-table entries a decode would
//                    read outside the page pool (the split kernel clamps them).
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
//     wave's Q slice: its 512 latent dims in 128 VGPRs for the whole work
//     item, its 64 RoPE dims in LDS.  Each lane then
//     holds 16 scores of ONE head, so max/sum need a single cross-lane step
//     (lane l ^ 32) and P is already laid out as the B operand of P·V.
//   * Output is also transposed, Oᵀ[v][h] += Vᵀ[v][n]·Pᵀ[n][h]: 16 MFMA tiles
//     of 32 value columns, accumulator 32 heads × 512 fp32 = 256 AGPRs; every
//     value a lane holds belongs to its own head, so rescaling is lane-local.
//     The Vᵀ operand is read straight from the row-major tile with gfx950's
//     transposing LDS read (ds_read_b64_tr_b16): no second copy of the tile.
//   * Cache rows go HBM -> LDS with global_load_lds_dwordx4 (no VGPRs): one
//     instruction moves one 1 KiB latent row (or eight 128-byte RoPE rows).
//     A ring of 4 tiles of 32 rows (36 KiB each): two tiles in flight, one
//     being scored, one being multiplied into the output; one barrier per tile.
//   * One wave per SIMD, so the loop is software-pipelined by hand: the score
//     MFMAs of tile t run with the softmax of tile t-1 placed between them,
//     then the P·V MFMAs of tile t-1; LDS operands are read three MFMAs ahead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_rule.h"
#include "mla_kernels.h"

#include <hip/hip_ext.h>

#include <mutex>

namespace mla {

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
__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}
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
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, h2));   // one v_cvt_pk_f16_f32
  } else {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
}

// Split partials: a row whose values all lie within [-kPart16Max,
// kPart16Max] is kept in fp16 only; a larger one in fp32 too.  The choice
// rides in the low mantissa bit of the row's base-2 lse (a change of one
// ulp; -inf, the empty split, has it clear).
constexpr float kPart16Max = 1.0f;
__device__ __forceinline__ float lse_with_flag(float lse2, bool big) {
  return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, lse2) & ~1u) | (big ? 1u : 0u));
}
__device__ __forceinline__ bool lse_flag(float raw) { return (__builtin_bit_cast(uint32_t, raw) & 1u) != 0; }
__device__ __forceinline__ float lse_value(float raw) {
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, raw) & ~1u);
}

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
constexpr int kStages = 4;                         // LDS ring of tiles (144 KiB)
constexpr int kLoadsPerTile = 9;                   // DMA instructions per wave per tile
constexpr int kXcds = 8;                           // accelerator complex dies, each with its own L2
constexpr int kQRegSteps = 32;                     // Q k-steps held in VGPRs (the latent part)
constexpr int kQLdsBytes = 4 * 4 * 1024;           // RoPE k-steps of Q: [step][wave][lane] x 16 B
static_assert(kStages * kTileBytes + kQLdsBytes <= 160 * 1024, "LDS budget of a gfx950 workgroup");

__device__ __forceinline__ int swz_lat(int n) { return ((n & 3) << 2) | ((n >> 2) & 3); }
__device__ __forceinline__ int swz_rope(int n) { return (n >> 1) & 7; }

// FP8 (E4M3) cache.  A tile arrives as bytes, [32][512] latent then [32][64]
// RoPE, in one of two staging slots, and each wave widens the rows it loaded
// itself into a 16-bit ring slot of the layout above (values as stored,
// exactly: every E4M3 value is an fp16 and a bf16 value), so that the
// products read the same operands as with a 16-bit cache.  The ring shrinks
// to three slots; the two staging slots take the fourth one's place.
constexpr int kLat8Bytes = kTileRows * 512;           // 16384
constexpr int kTile8Bytes = kLat8Bytes + kTileRows * 64;   // 18432
constexpr int kStages8 = 3;                           // 16-bit ring slots with an FP8 cache
constexpr int kStaging8 = kStages8 * kTileBytes;      // first staging slot
constexpr int kLoadsPerTile8 = 6;                     // DMA instructions per wave per FP8 tile
static_assert(kStaging8 + 2 * kTile8Bytes == kStages * kTileBytes, "FP8 staging fills the fourth ring slot");

typedef short s16x4 __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) char lds_char;
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

// s_waitcnt on the vector-memory counter (VM) and the LDS/scalar-memory
// counter (LGKM, 15 = no constraint); gfx9 encoding.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_cnt() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (LGKM << 8));
}

// Barrier without a memory fence: cross-wave data in the loop are DMA tiles,
// whose arrival every wave waits for explicitly before it.  The "memory"
// clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Fence for the instruction scheduler: nothing moves across it.  The loop
// below places one MFMA per fenced region together with the LDS reads and the
// softmax instructions that are to run while that MFMA occupies the matrix
// core; a wave per SIMD has no other wave to hide its latencies.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ u32x4 lds_get16(const lds_char* base, int byte_off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base + byte_off);
}

// Two transposing reads give the 8 contraction values of one A operand.
__device__ __forceinline__ u32x4 lds_get_tr(const lds_char* b0, int off0, const lds_char* b1, int off1) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(b0 + off0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(b1 + off1));
  u32x2 a2 = __builtin_bit_cast(u32x2, a), b2 = __builtin_bit_cast(u32x2, b);
  return u32x4{a2.x, a2.y, b2.x, b2.y};
}

// max of three floats in one VALU op (fmaxf would first canonicalise each
// input, as the compiler cannot see that the scores are not signalling NaNs).
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max(a, |b|, |c|) in one VALU op (operand modifiers).
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// ---------------------------------------------------------------------------
// Split planner inside the split kernel
// ---------------------------------------------------------------------------
// In planner mode every wave of the main pass runs the planner rule of
// plan_rule.h itself, on one wave with no barrier: the same integers as the
// host twin and the stand-alone planner kernel.  This saves a kernel launch
// per call.  Workgroup 0 publishes the plan (num_splits, split_offset, work)
// for the combine kernel.

// Sum and max over the 64 lanes: DPP within each row of 16 lanes (pairs,
// quads, halves, rows), then the four row results through readlane.  Every
// lane must be active.
__device__ __forceinline__ int row_sum_i32(int v) {
  v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);   // row_half_mirror
  v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);   // row_mirror
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  v = row_sum_i32(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
// Sum of a 64-bit value over the lanes: three 16-bit slices summed with
// wave_sum_i32 (each slice sum stays below 2^22 in 32 bits), recombined;
// for the per-lane sums the planner forms (below 2^46).
__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
  const int lo = wave_sum_i32((int)(v & 0xFFFF));
  const int mid = wave_sum_i32((int)((v >> 16) & 0xFFFF));
  const int hi = wave_sum_i32((int)(v >> 32));
  return ((int64_t)hi << 32) + ((int64_t)mid << 16) + (int64_t)lo;
}
// Inclusive prefix sum over the 64 lanes with DPP: within each row of 16
// lanes by shifts of 1, 2, 4 and 8 (a lane shifted in from outside the row
// adds 0), then across rows: row_bcast:15 adds the last lane of rows 0 and 2
// to rows 1 and 3, row_bcast:31 adds lane 31 (rows 0 + 1) to rows 2 and 3.
// Every lane must be active.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31, rows 2 and 3
  return v;
}
// A value of lane `src` (wave-uniform) in every lane.
__device__ __forceinline__ int lane_value(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

struct WorkItem {
  int b, k, r0, r1, s_b;
  int slot;     // split slot (sequence-major: split_offset[b] + k)
  bool valid;   // false: past the last work item of the plan
};

// Work item wi of a plan made beforehand (split_kernel's GIVEN instances;
// device data, not checked on the host): the work list is in slot order,
// and num_cus holds the plan's capacity.  Every field is
// clamped, so that a plan that does not match the lengths gives wrong rows,
// never an access outside the buffers.
__device__ __forceinline__ WorkItem given_item(const SplitParams& p, int wi) {
  WorkItem it{};
  it.valid = wi < min(p.split_offset[p.batch], p.num_cus);
  if (!it.valid) return it;
  const int32_t* w = p.work + 4 * (int64_t)wi;
  it.b = min(max(w[0], 0), p.batch - 1);
  const int L = clamp_len(p.seqlens[it.b], p.row_cap);
  it.s_b = max(p.num_splits[it.b], 1);
  it.k = min(max(w[1], 0), it.s_b - 1);
  it.r0 = min(max(w[2], 0), L);
  it.r1 = min(max(w[3], it.r0), L);
  it.slot = wi;
  return it;
}

// Sequences per lane whose lengths the planner keeps in registers (batch <=
// 256); larger batches re-read the lengths where they need them.
constexpr int kPlanRegs = 4;

__device__ WorkItem plan_item(const SplitParams& p, int wi, int lane, bool publish) {
  const int B = p.batch;
  // Lane l owns the contiguous sequences [b0, b1); per is uniform.
  const int per = (B + 63) / 64;
  const int b0 = min(B, lane * per), b1 = min(B, b0 + per);
  const bool in_regs = per <= kPlanRegs;
  int Lr[kPlanRegs];   // clamped lengths of the lane's sequences
#pragma unroll
  for (int j = 0; j < kPlanRegs; ++j) {
    Lr[j] = -1;
    if (in_regs && j < per && b0 + j < b1) Lr[j] = clamp_len(p.seqlens[b0 + j], p.row_cap);
  }
  // Length of the lane's j-th sequence b = b0 + j (-1 past its last).
  auto len_of = [&](int j, int b) __attribute__((always_inline)) -> int {
    if (in_regs) {
      int L = -1;
#pragma unroll
      for (int jj = 0; jj < kPlanRegs; ++jj)
        if (jj == j) L = Lr[jj];
      return L;
    }
    return clamp_len(p.seqlens[b], p.row_cap);
  };
  const int sq = p.seqlen_q, tail = tail_splits(sq);
  // Blocks of the prefix of a sequence of L rows (the part the budget cuts).
  auto pre_blocks = [&](int L) __attribute__((always_inline)) { return num_blocks(prefix_len(L, sq)); };
  // Prefix splits of the lane's sequences under budget t (the budget bounds
  // these; the tails come on top).
  auto lane_splits = [&](int t) __attribute__((always_inline)) -> int {
    int cnt = 0;
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < kPlanRegs; ++j)
        if (j < per) cnt += Lr[j] >= 0 ? splits_for_budget(pre_blocks(Lr[j]), t) : 0;
    } else {
      for (int b = b0; b < b1; ++b) cnt += splits_for_budget(pre_blocks(clamp_len(p.seqlens[b], p.row_cap)), t);
    }
    return cnt;
  };
  int maxnb = 0;
  int64_t sumnb = 0;
  if (in_regs) {
#pragma unroll
    for (int j = 0; j < kPlanRegs; ++j)
      if (j < per) {
        const int nb = Lr[j] >= 0 ? pre_blocks(Lr[j]) : 0;
        maxnb = max(maxnb, nb);
        sumnb += nb;
      }
  } else {
    for (int b = b0; b < b1; ++b) {
      const int nb = pre_blocks(clamp_len(p.seqlens[b], p.row_cap));
      maxnb = max(maxnb, nb);
      sumnb += nb;
    }
  }
  maxnb = wave_max_i32(maxnb);
  sumnb = wave_sum_i64(sumnb);
  // Smallest budget t with sum_b splits_for_budget(nb_b, t) <= cap; the sum
  // is at least sum_b nb_b / t, so t starts at ceil(sum nb / cap).
  const int cap = planner_cap(B, p.heads, p.num_cus, sq);
  int hi = maxnb > 1 ? maxnb : 1;
  const int64_t lo64 = sumnb < (1 << 30) && cap < (1 << 30) ? ceil_div_small((int)sumnb, cap) : (sumnb + cap - 1) / cap;
  int lo = (int)(lo64 < 1 ? 1 : (lo64 > hi ? hi : lo64));
  // Equal lengths meet the cap at the lower bound: one probe instead of a search.
  if (lo < hi && wave_sum_i32(lane_splits(lo)) <= cap) hi = lo;
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    if (wave_sum_i32(lane_splits(mid)) <= cap) hi = mid;
    else lo = mid + 1;
  }
  const int t = lo;
  const int mine = lane_splits(t) + tail * (b1 - b0);   // all splits of the lane's sequences
  const int incl = wave_incl_scan(mine);
  const int off = incl - mine;
  const int total = lane_value(incl, 63);
  if (publish) {
    int o = off;
    for (int b = b0; b < b1; ++b) {
      const int L = clamp_len(p.seqlens[b], p.row_cap);
      const int spre = splits_for_budget(pre_blocks(L), t), sb = spre + tail;
      p.num_splits[b] = sb;
      p.split_offset[b] = o;
      for (int k = 0; k < sb; ++k) {
        int r0, r1;
        seq_split_range(L, sq, spre, k, &r0, &r1);
        int* w = p.work + 4 * (o + k);
        w[0] = b;
        w[1] = k;
        w[2] = r0;
        w[3] = r1;
      }
      o += sb;
    }
    if (lane == 63) p.split_offset[B] = total;
  }
  WorkItem it{};
  it.valid = wi < total;
  if (!it.valid) return it;
  // Work-item order (not slot order): with several query tokens the 2B tail
  // splits first (item wi < 2B: sequence wi / 2, tail wi % 2), then the
  // prefix splits in sequence order; the split kernel deals the two kinds to
  // the XCDs separately.  Split slots stay sequence-major.
  const int ntail = tail * B;
  int owner, j = 0;
  if (wi < ntail) {
    owner = (wi / tail) / per;   // the lane holding sequence wi / tail
  } else {
    j = wi - ntail;              // the j-th prefix split
    const int mine_pre = mine - tail * (b1 - b0);
    const int off_pre = wave_incl_scan(mine_pre) - mine_pre;
    owner = __builtin_ctzll(__ballot(j >= off_pre && j < off_pre + mine_pre));
    j -= lane_value(off_pre, owner);
  }
  int fb = 0, fk = 0, fL = 0, fslot = 0;
  if (lane == owner) {
    int o = off, jj = j;
    for (int b = b0; b < b1; ++b) {
      const int L = len_of(b - b0, b);
      const int spre = splits_for_budget(pre_blocks(L), t);
      if (wi < ntail ? b == wi / tail : jj < spre) {
        fb = b;
        fk = wi < ntail ? spre + wi % tail : jj;
        fL = L;
        fslot = o + fk;
        break;
      }
      jj -= spre;
      o += spre + tail;
    }
  }
  it.b = lane_value(fb, owner);
  it.k = lane_value(fk, owner);
  it.slot = lane_value(fslot, owner);
  const int L = lane_value(fL, owner);
  const int spre = splits_for_budget(pre_blocks(L), t);
  it.s_b = spre + tail;
  seq_split_range(L, sq, spre, it.k, &it.r0, &it.r1);
  return it;
}

// ---------------------------------------------------------------------------
// Split kernel
// ---------------------------------------------------------------------------

// One direct-to-LDS load: 64 lanes x 16 bytes from base + (lane16 ^ key)
// (per lane) into the 1 KiB of LDS at lds_addr (lane l -> lds_addr + 16 l).
// Issued through inline asm so that the compiler does not add its own
// conservative waits for the LDS write before every LDS read; the
// vector-memory counter is managed explicitly (wait_cnt).  The lane offset is
// formed inside the asm so that it cannot be hoisted out of the loop into a
// register of its own.  One wait state separates the M0 write from the load
// that reads it.
__device__ __forceinline__ void dma16(const void* base, uint32_t lane16, uint32_t key, uint32_t lds_addr) {
  uint32_t voff;
  asm volatile("v_xor_b32 %0, %1, %2\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %4"
               : "=&v"(voff)
               : "s"(key), "v"(lane16), "s"(lds_addr), "s"(base)
               : "memory");
}

// The RoPE load of a tile: lane l carries 16 bytes of row n = 8w + l/8
// (clamped to nlast) at slot (l % 8) ^ swz_rope(n), from base + nn*rb +
// 16 ((l % 8) ^ ((n / 2) % 8)) into lds_addr + 16 l.  Everything per lane is
// formed inside the asm from the lane id (v_mbcnt), for the reason given
// above and to hold no register across the loop.  w8 = 8w.
__device__ __forceinline__ void dma16_rope(const void* base, int w8, int nlast, uint32_t rb, uint32_t lds_addr) {
  uint32_t l, n, t;
  asm volatile(
      "v_mbcnt_lo_u32_b32 %0, -1, 0\n\t"
      "v_mbcnt_hi_u32_b32 %0, -1, %0\n\t"       // l = lane id
      "v_lshrrev_b32 %1, 3, %0\n\t"
      "v_add_u32 %1, %3, %1\n\t"                // n = 8w + l/8
      "v_lshrrev_b32 %2, 1, %1\n\t"
      "v_xor_b32 %2, %2, %0\n\t"
      "v_and_b32 %2, 7, %2\n\t"
      "v_lshlrev_b32 %2, 4, %2\n\t"             // t = 16 ((l ^ n/2) % 8)
      "v_min_i32 %1, %4, %1\n\t"
      "v_mad_u32_u24 %1, %1, %5, %2\n\t"        // nn*rb + t (nn < 32, rb < 2^24)
      "s_mov_b32 m0, %6\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %7"
      : "=&v"(l), "=&v"(n), "=&v"(t)
      : "s"(w8), "s"(nlast), "s"(rb), "s"(lds_addr), "s"(base)
      : "memory");
}

// FP8 tile loads.  Latent: one instruction moves two 512-byte rows, lane l
// carrying bytes 16 (l % 32) .. + 15 of row n0 + l / 32 into lds_addr + 16 l;
// base is row n0 (already clamped) and hi_off the byte offset of the second
// row from it (0 when that row is past the last valid one, which is then
// re-read).  RoPE: one 4-byte instruction moves four 64-byte rows, lane l
// carrying bytes 4 (l % 16) .. + 3 of row n0 + l / 16 (clamped to nlast) into
// lds_addr + 4 l.  Per-lane offsets are formed inside the asm, as in dma16.
__device__ __forceinline__ void dma8_lat(const void* base, uint32_t hi_off, uint32_t lane16, uint32_t lds_addr) {
  uint32_t voff, h;
  asm volatile(
      "v_and_b32 %0, 0x1f0, %2\n\t"            // 16 (l % 32)
      "v_bfe_u32 %1, %2, 9, 1\n\t"              // l / 32
      "v_mad_u32_u24 %0, %1, %3, %0\n\t"
      "s_mov_b32 m0, %4\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %5"
      : "=&v"(voff), "=&v"(h)
      : "v"(lane16), "s"(hi_off), "s"(lds_addr), "s"(base)
      : "memory");
}
__device__ __forceinline__ void dma8_rope(const void* base, int n0, int nlast, uint32_t rb, uint32_t lds_addr) {
  uint32_t l, n;
  asm volatile(
      "v_mbcnt_lo_u32_b32 %0, -1, 0\n\t"
      "v_mbcnt_hi_u32_b32 %0, -1, %0\n\t"       // l = lane id
      "v_lshrrev_b32 %1, 4, %0\n\t"
      "v_add_u32 %1, %2, %1\n\t"                // n = n0 + l/16
      "v_min_i32 %1, %3, %1\n\t"
      "v_and_b32 %0, 15, %0\n\t"
      "v_lshlrev_b32 %0, 2, %0\n\t"             // 4 (l % 16)
      "v_mad_u32_u24 %1, %1, %4, %0\n\t"        // nn*rb + 4 (l % 16) (nn < 32, rb < 2^24)
      "s_mov_b32 m0, %5\n\ts_nop 0\n\t"
      "global_load_lds_dword %1, %6"
      : "=&v"(l), "=&v"(n)
      : "s"(n0), "s"(nlast), "s"(rb), "s"(lds_addr), "s"(base)
      : "memory");
}

// Two E4M3 values (the low or the high byte pair of w, lowest byte first)
// widened to the 16-bit type DT in one instruction, v_cvt_scalef32_pk_*_fp8
// with scale 1: exact, as every E4M3 value is an fp16 and a bf16 value, and
// the E4M3 NaN codes give NaN.  Written as asm: the compiler's own lowering
// of the builtin extracted the second half of the result wrongly (both
// halves came out as the first byte's value).
template <int DT, bool HI>
__device__ __forceinline__ uint32_t widen2(uint32_t w) {
  uint32_t r;
  if constexpr (DT == MLA_DTYPE_F16) {
    if constexpr (HI) asm("v_cvt_scalef32_pk_f16_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(r) : "v"(w));
    else asm("v_cvt_scalef32_pk_f16_fp8 %0, %1, 1.0" : "=v"(r) : "v"(w));
  } else {
    if constexpr (HI) asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(r) : "v"(w));
    else asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0" : "=v"(r) : "v"(w));
  }
  return r;
}

// sbase + (lane_bits ^ key): per-tile LDS read addresses (sbase = the tile's
// slot, lane_bits = this lane's loop-invariant offset bits, key = the part
// that varies with the operand).  asm volatile keeps the compiler from
// hoisting one register per operand offset out of the loop.
__device__ __forceinline__ uint32_t xor_add(uint32_t sbase, uint32_t key, uint32_t lane_bits) {
  uint32_t r;
  asm volatile("v_xor_b32 %0, %1, %2\n\tv_add_u32 %0, %3, %0" : "=&v"(r) : "s"(key), "v"(lane_bits), "s"(sbase));
  return r;
}


__device__ __forceinline__ const lds_char* lds_at(uint32_t addr) {
  return (const lds_char*)(uintptr_t)addr;
}

__device__ __forceinline__ uint32_t lds_u32(const lds_char* p) { return (uint32_t)(uintptr_t)p; }

// Where the work item's cache rows live, and the next tile to load (all
// wave-uniform).  Tiles are loaded in order, 32 rows apart; a tile (32 rows at
// a multiple of 32) never straddles a page, since pages hold a multiple of 32
// rows, so a paged tile is one page index plus a row offset inside the page.
struct DmaCursor {
  const char* lat;      // contiguous: latent row `row`; paged: the pool
  const char* rope;     // likewise for the RoPE part
  const_i32_ptr bt;     // paged: the block-table entry of the next tile
  int64_t lat_pb, rope_pb;    // paged: page strides in bytes
  uint32_t lat_rb, rope_rb;   // row strides in bytes
  int page_size, num_pages;
  int row;                    // first logical row of the next tile
  int in_page;                // paged: its row inside the page
};

// Physical page of the cursor's tile (paged), clamped to the pool.  A scalar
// load: the block table is read-only for the kernel.
__device__ __forceinline__ int cursor_page(const DmaCursor& c) {
  const int pg = *c.bt;
  return pg < 0 ? 0 : (pg >= c.num_pages ? c.num_pages - 1 : pg);
}

// One tile's load: base of its row 0 (latent and RoPE) and its last valid row.
struct DmaTile {
  const char* lat;
  const char* rope;
  int nlast;            // rows at or past it re-read it (0 <= nlast)
  uint32_t lds;         // the tile's LDS slot
};

template <bool PAGED>
__device__ __forceinline__ DmaTile cursor_tile(const DmaCursor& c, int page, int r1, const lds_char* tile) {
  DmaTile d;
  if constexpr (PAGED) {
    d.lat = c.lat + page * c.lat_pb + (int64_t)c.in_page * c.lat_rb;
    d.rope = c.rope + page * c.rope_pb + (int64_t)c.in_page * c.rope_rb;
  } else {
    d.lat = c.lat;
    d.rope = c.rope;
  }
  d.nlast = r1 - 1 - c.row;
  d.lds = lds_u32(tile);
  return d;
}

// Next tile, except that the cursor stays on the work item's last tile (the
// one holding row r1 - 1): the loop loads a tile every step, and past the end
// it reloads that last tile (valid memory) into a slot nothing reads again.
// Branch-free (a branch here splits the loop body and costs register copies
// at the join).
template <bool PAGED>
__device__ __forceinline__ void cursor_next(DmaCursor& c, int r1) {
  const int adv = c.row + kTileRows < r1 ? 1 : 0;
  c.row += adv * kTileRows;
  if constexpr (PAGED) {
    c.in_page += adv * kTileRows;
    const int wrap = c.in_page == c.page_size ? 1 : 0;
    c.in_page -= wrap * c.page_size;
    c.bt += wrap;
  } else {
    c.lat += (int64_t)(adv * kTileRows) * c.lat_rb;
    c.rope += (int64_t)(adv * kTileRows) * c.rope_rb;
  }
}

// This wave's part of a tile load: part 0 moves the RoPE parts of rows
// 8w .. 8w+7 (first, so that its base register is free early), part i >= 1
// latent row 8w + i - 1.  Rows past nlast re-read row nlast (always valid);
// their scores are masked.
__device__ __forceinline__ void issue_part(const DmaCursor& c, const DmaTile& d, int wave, uint32_t lane16,
                                           int part) {
  if (part > 0) {
    const int n = 8 * wave + part - 1;
    const int nn = n < d.nlast ? n : d.nlast;
    dma16(d.lat + (uint32_t)nn * c.lat_rb, lane16, (uint32_t)(16 * swz_lat(n)), d.lds + n * 1024);
  } else {
    // lane l carries row 8w + l/8, slot l % 8 (holding chunk slot ^ swz_rope(row))
    dma16_rope(d.rope, 8 * wave, d.nlast, c.rope_rb, d.lds + kLatBytes + 8 * wave * 128);
  }
}

// This wave's part of an FP8 tile load into a staging slot: parts 0..3 the
// latent rows 8w + 2 part, + 1 (staged row n at 512 n), parts 4 and 5 the RoPE
// rows 8w + 4 (part - 4) .. + 3 (staged row n at kLat8Bytes + 64 n).  Rows
// past nlast re-read row nlast.
__device__ __forceinline__ void issue_part8(const DmaCursor& c, const DmaTile& d, int wave, uint32_t lane16,
                                            int part) {
  if (part < 4) {
    const int n = 8 * wave + 2 * part;
    const int nn = n < d.nlast ? n : d.nlast;
    const uint32_t hi = n + 1 <= d.nlast ? c.lat_rb : 0u;
    dma8_lat(d.lat + (uint32_t)nn * c.lat_rb, hi, lane16, d.lds + 1024 * (4 * wave + part));
  } else {
    const int j = part - 4;
    dma8_rope(d.rope, 8 * wave + 4 * j, d.nlast, c.rope_rb, d.lds + kLat8Bytes + 256 * (2 * wave + j));
  }
}

// Widening of an FP8 tile, this wave's share: the bytes its own loads
// staged (so only its own load counter guards them, no barrier).  Nine
// 16-byte chunks of the 16-bit ring slot per lane: for u = 0..3 the staged
// 16 bytes at 1024 (4w + u) + 16 l, i.e. values 16 (l % 32) .. + 15 of latent
// row n = 8w + 2u + l/32, become chunks 2 (l % 32) and 2 (l % 32) + 1 of that
// row; then the staged RoPE bytes at kLat8Bytes + 512 w + 8 l, values
// 8 (l % 8) .. + 7 of RoPE row 8w + l/8, become that row's chunk l % 8.
// Ring positions follow the swizzles above, split into a per-lane part and a
// wave-uniform key (disjoint bits, so xor and add agree):
//   latent chunk 2 (l % 32) + e of row n: 8192 w + 2048 u + (lat8_lane ^ 16 k),
//     lat8_lane = 1024 (l/32) + 16 (2 (l % 32) ^ 4 (l/32)),
//     k = 8 (u % 2) ^ ((2w + u/2) % 4) ^ e;
//   RoPE chunk l % 8 of row 8w + l/8: kLatBytes + 1024 w + (rope8_lane ^ 64 (w % 2)),
//     rope8_lane = 128 (l/8) + 16 ((l % 8) ^ (l/16)).
__device__ __forceinline__ uint32_t lat8_lane(uint32_t lane) {
  const uint32_t h = lane >> 5;
  return 1024u * h + 16u * ((2u * (lane & 31u)) ^ (4u * h));
}
__device__ __forceinline__ uint32_t rope8_lane(uint32_t lane) {
  return 128u * (lane >> 3) + 16u * ((lane & 7u) ^ (lane >> 4));
}
__device__ __forceinline__ uint32_t lat8_key(int wave, int u, int e) {
  return 16u * (uint32_t)((8 * (u & 1)) ^ ((2 * wave + (u >> 1)) & 3) ^ e);
}


// Softmax of one score tile, cut into steps so that the loop can run them one
// or two instructions at a time between MFMAs.  x[] holds the raw scores
// (q·k, not yet scaled) of this lane's head; the steps turn them into
// P = 2^(c x - c m) and pack P as the B operand of P·V.  c = softmax_scale ·
// log2(e) > 0, so the max of the raw scores is the max of the scaled ones.
//
// The reference max `m` is taken from the work item's first tile and then
// changed only when a later tile's max passes it by more than kRescaleMargin
// (log2 units): P = 2^(c x - c m) may exceed 1, which is exact while it stays
// inside the range of the P·V operand type.  Step 5 leaves dn = c m - c
// tmax (<= 0 when the tile's max is higher); raising m means scaling the
// accumulator (all 256 AGPRs of the lane) and the running sum by alpha =
// 2^dn, which the loop does in a rarely taken branch right after step 5,
// before this tile's exponentials and sums.  Only nmc = -c m is kept.
//
// Two running sums of P: `lsum` of the fp32 values (it gives the split's
// log-sum-exp, hence the weights between splits) and, for fp16, `lsr` of the
// values as rounded for the P·V product (one v_dot2c per packed pair).  The
// split's output is normalised by lsr, so that it is exactly a convex
// combination of value rows under the weights actually multiplied: the
// rounding of a dominant P then cancels.  (The lse from lsr too would carry
// P's rounding, up to 2^-11 relative, into the weights between splits,
// where large value rows of two splits that cancel amplify it.)  bf16 keeps
// P as hi + lo (relative error 2^-17), so lsum serves both.
template <int DT>
constexpr float kRescaleMargin = DT == MLA_DTYPE_F16 ? 15.0f : 64.0f;

template <int DT>
struct Softmax {
  float x[16];
  float t0, t1, t2, t3, t4, tmax;
  float dn;             // step 5: c m - c tmax (0 on the first tile)
  u32x4 pk[2], pl[2];   // P packed (bf16: high part in pk, low part in pl)

  // Step `s` (0 .. kSoftmaxSteps<DT> - 1).  `first`: this is the work item's
  // first tile, which fixes m.
  __device__ __forceinline__ void step(int s, bool first, float c, float& nmc, float& lsum, float& lsr) {
    if (s == 0) { t0 = max3(x[0], x[1], x[2]); t1 = max3(x[3], x[4], x[5]); }
    if (s == 1) { t2 = max3(x[6], x[7], x[8]); t3 = max3(x[9], x[10], x[11]); }
    if (s == 2) { t4 = max3(x[12], x[13], x[14]); t0 = max3(t0, t1, x[15]); }
    if (s == 3) { tmax = max3(t0, t2, t3); tmax = max3(tmax, t4, t4); }
    if (s == 4) {
      float a = tmax, b = tmax;
      swap_halves(a, b);
      tmax = max3(a, b, b);
    }
    if (s == 5) {
      if (first) {
        // A query row with no visible row in the first tile (possible in a
        // tail split) has tmax = -inf: it uses 0 as the max, so that P =
        // 2^-inf = 0 rather than 2^(-inf + inf).
        nmc = tmax == -__builtin_inff() ? 0.f : -(tmax * c);
        dn = 0.f;
      } else {
        dn = __builtin_fmaf(tmax, -c, -nmc);   // -inf max: +inf, no rescale
      }
    }
    if (s >= 6 && s < 22) {
      const int e = s - 6;
      x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], c, nmc));
    }
    if (s >= 7 && s < 23) lsum += x[s - 7];
    if (s >= 8 && s < 23 && (s & 1) == 0) {
      const int j = (s - 8) >> 1;   // pair j = exponentials 2j, 2j+1
      const float a = x[2 * j], bb = x[2 * j + 1];
      const uint32_t w = pack2<DT>(a, bb);
      pk[j >> 2][j & 3] = w;
      if constexpr (DT == MLA_DTYPE_F16) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        lsr = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, w), (h2){(_Float16)1.0f, (_Float16)1.0f}, lsr, false);
      }
    }
    // bf16: the low part of pair j, in steps 23..30, which the score MFMAs
    // of the loop would otherwise pass with only their K reads between them.
    if constexpr (DT == MLA_DTYPE_BF16) {
      if (s >= 23 && s < 31) {
        const int j = s - 23;
        const uint32_t w = pk[j >> 2][j & 3];
        const float a = x[2 * j], bb = x[2 * j + 1];
        const float ah = __builtin_bit_cast(float, w << 16);
        const float bh = __builtin_bit_cast(float, w & 0xFFFF0000u);
        pl[j >> 2][j & 3] = pack2<DT>(a - ah, bb - bh);
      }
    }
  }
};
template <int DT>
constexpr int kSoftmaxSteps = DT == MLA_DTYPE_BF16 ? 31 : 23;

// Schedule (one wave, work item of n tiles; tile t in LDS slot t % 4):
//   prologue   DMA tiles 0, 1, 2; wait for tile 0; barrier
//   step t     A: the 36 score MFMAs of tile t, with the softmax of tile t-1
//                 run between them (steps of Softmax), K reads ahead;
//              B: the P·V MFMAs of tile t-1, V reads ahead, and this wave's
//                 9 loads of tile t+2 (into tile t-2's slot), one every three
//                 MFMAs;
//              before its last few MFMAs: wait until tile t+1 has landed and
//                 every wave has finished reading tile t-1, then start the K
//                 reads of tile t+1.
//   drain      softmax of tile n-1 (masked), P·V of tile n-1.
// Two tiles stay in flight, one barrier per tile; only the last tile can be
// partial, so masking is confined to the drain.
// GIVEN: the work items come from a plan made beforehand (given_item), an
// instance of its own so that the other instances keep their registers.
template <int DT, bool PAGED, bool KV8, bool GIVEN>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void split_kernel(SplitParams p) {
  constexpr int EB = KV8 ? 1 : 2;   // bytes per cache element
  __shared__ __attribute__((aligned(1024))) char lds_raw[kStages * kTileBytes + kQLdsBytes];
  lds_char* lds = (lds_char*)lds_raw;
  lds_char* qlds = lds + kStages * kTileBytes;

  // Workgroup -> (work item, head group).  The dispatcher deals workgroups to
  // the 8 XCDs round-robin by flat id; this bijection gives each XCD a
  // contiguous run of (work item, head group) pairs in work-item-major order,
  // so that the splits of a sequence share one L2 for their queries, and the
  // head groups of a work item its cache rows.
  //
  // With several query tokens the workgroups come in two kinds (a plan made
  // beforehand lists them in slot order and takes the plain bijection),
  // the full-length prefix splits and the one-tile tails (work items below
  // tail * B, see plan_item); each XCD gets an even share of each kind, the
  // prefix splits first, so that the two head groups of a split start
  // together and no XCD queues a full-length split behind another.  With one
  // token this is the plain bijection above.
  int wi, hg;
  {
    const int ng = gridDim.y;
    const int total = gridDim.x * ng;
    const int flat = blockIdx.x + blockIdx.y * gridDim.x;
    const int xcd = flat & (kXcds - 1), idx = flat / kXcds;
    const int nt = GIVEN ? 0 : tail_splits(p.seqlen_q) * p.batch * ng;   // tail workgroups
    const int nb = total - nt;                                         // the others
    // Workgroups of each kind before XCD x, and on XCD x.
    auto before = [&](int n, int x) { return x * (n / kXcds) + min(x, n % kXcds); };
    const int nb_x = before(nb, xcd + 1) - before(nb, xcd);
    int lin;
    if (idx < nb_x) {
      lin = nt + before(nb, xcd) + idx;
    } else {   // XCD x's tails: the rest of its workgroups (never negative)
      lin = (before(total, xcd) - before(nb, xcd)) + (idx - nb_x);
    }
    wi = lin / ng;
    hg = lin - wi * ng;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hl = lane & 31;
  const int g = lane >> 5;
  const uint32_t lane16 = 16u * (uint32_t)lane;

  // ---- work item (uniform) -------------------------------------------------
  // k: the split's index within its sequence; with several query tokens the
  // last two splits are the tails, whose rows are masked per query row.
  // split_slot (sequence-major) indexes the partials; with tails, work items
  // come tails first (see plan_item).
  int b, k, r0, r1, s_b, split_slot = wi;
  if (p.num_split > 0) {
    s_b = p.num_split;
    const int tl = tail_splits(p.seqlen_q), pre = s_b - tl;
    if (tl > 0) {
      if (wi < tl * p.batch) {
        b = wi / tl;
        k = pre + wi % tl;
      } else {
        b = (wi - tl * p.batch) / pre;
        k = (wi - tl * p.batch) - b * pre;
      }
      split_slot = b * s_b + k;
    } else {
      b = wi / s_b;
      k = wi - b * s_b;
    }
    seq_split_range(clamp_len(p.seqlens[b], p.row_cap), p.seqlen_q, pre, k, &r0, &r1);
  } else {
    WorkItem it;
    if constexpr (GIVEN) it = given_item(p, wi);
    else it = plan_item(p, wi, lane, wi == 0 && hg == 0 && wave == 0);
    if (!it.valid) return;   // past the end of the plan
    b = it.b;
    k = it.k;
    r0 = it.r0;
    r1 = it.r1;
    s_b = it.s_b;
    split_slot = it.slot;
  }
  // Tail splits (the last two with several query tokens): query token t sees
  // rows j < L - (seqlen_q - 1 - t) = tail_lim + t.  Other splits: no limit.
  int tail_lim = INT32_MAX;
  if (p.seqlen_q > 1 && k >= s_b - tail_splits(p.seqlen_q))
    tail_lim = clamp_len(p.seqlens[b], p.row_cap) - (p.seqlen_q - 1);
  tail_lim = __builtin_amdgcn_readfirstlane(tail_lim);
  split_slot = __builtin_amdgcn_readfirstlane(split_slot);
  b = __builtin_amdgcn_readfirstlane(b);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  r1 = __builtin_amdgcn_readfirstlane(r1);
  s_b = __builtin_amdgcn_readfirstlane(s_b);
  const int n_tiles = (r1 - r0 + kTileRows - 1) / kTileRows;

  // Heads of this wave.  Lanes past the last head compute with a zero query
  // and write nothing.
  const int h0 = hg * kHeadsPerGroup + wave * 32;
  const bool head_ok = h0 + hl < p.heads;
  const int h = head_ok ? h0 + hl : p.heads - 1;

  u32x4 qreg[kQRegSteps];
  // This wave's Q RoPE slots: qlds + 1024 wave + 16 lane (+ 4096 per k-step).
  const uint32_t qwave = lds_u32(qlds) + 1024u * (uint32_t)wave;

  DmaCursor cur;
  cur.lat_rb = (uint32_t)(p.kv_sr * EB);
  cur.rope_rb = (uint32_t)(p.kpe_sr * EB);
  cur.row = r0;
  if constexpr (PAGED) {
    cur.lat = reinterpret_cast<const char*>(p.kv);
    cur.rope = reinterpret_cast<const char*>(p.kpe);
    const int slot0 = r0 / p.page_size;
    cur.bt = (const_i32_ptr)(p.block_table + (int64_t)b * p.bt_stride + slot0);
    cur.lat_pb = p.kv_sb * EB;
    cur.rope_pb = p.kpe_sb * EB;
    cur.page_size = p.page_size;
    cur.num_pages = p.num_pages;
    cur.in_page = r0 - slot0 * p.page_size;
  } else {
    cur.lat = reinterpret_cast<const char*>(p.kv) + (int64_t)b * p.kv_sb * EB + (int64_t)r0 * cur.lat_rb;
    cur.rope = reinterpret_cast<const char*>(p.kpe) + (int64_t)b * p.kpe_sb * EB + (int64_t)r0 * cur.rope_rb;
  }

  // LDS byte offsets inside a tile, as loop-invariant lane bits plus a key
  // (disjoint bit ranges, so xor and add agree):
  //   score operand, k-step s < 32 (row hl, chunk 2s + g):
  //     hl*1024 + 256 (s / 8) + 16 ((2 (s % 8)) ^ kx), kx = g ^ swz_lat(hl)
  //     = (klx ^ 32 (s % 8)) + 256 (s / 8),   klx = hl*1024 | 16 kx;
  //   RoPE k-step 32 + u (chunk 2u + g):
  //     kLatBytes + hl*128 + 16 ((2u + g) ^ swz_rope(hl)) = rkx ^ 32u;
  //   transposing value read for column block vb, k-step kt, half r:
  //     (vofs0 ^ 32 r ^ 64 (vb % 4)) + 256 (vb / 4) + 16384 kt + 8192 r.
  const uint32_t klx = (uint32_t)(hl * 1024) | (uint32_t)(16 * (g ^ swz_lat(hl)));
  const uint32_t rkx = (uint32_t)(kLatBytes + hl * 128) | (uint32_t)(16 * (g ^ swz_rope(hl)));
  // vofs1 = vofs0 ^ 32: the two halves differ only in z's bit 1.
  uint32_t vofs0;
  {
    const int i = lane & 15, G = lane >> 4;
    const int y = 2 * (G & 1) + ((i >> 1) & 1);
    const int z = (G >> 1) & 3;
    vofs0 = 4096 * (G >> 1) + 1024 * (i >> 2) + 64 * (i >> 2) + 16 * (y ^ z) + 8 * (i & 1);
  }
  // Ring slot of tile t (16-bit operands), and with an FP8 cache the staging
  // slot its bytes arrive in.
  auto slot = [&](int t) __attribute__((always_inline)) -> lds_char* {
    if constexpr (KV8) return lds + (t % kStages8) * kTileBytes;
    return lds + (t & (kStages - 1)) * kTileBytes;
  };
  auto stage8 = [&](int t) __attribute__((always_inline)) -> lds_char* { return lds + kStaging8 + (t & 1) * kTile8Bytes; };

  const float c = p.scale_log2;

  // An empty work item (more splits than blocks, or L = 0) writes out = 0 /
  // lse = -inf (or a zero partial, lse = -inf) and leaves before the
  // accumulator exists, so that it has a single definition path.
  if (n_tiles == 0) {
    if (!head_ok) return;
    if (s_b == 1) {
      uint16_t* o = p.out + (int64_t)b * p.out_sb + (int64_t)h * p.out_sh + 4 * g;
#pragma unroll
      for (int k = 0; k < 64; ++k) *reinterpret_cast<u32x2*>(o + 8 * k) = u32x2{0u, 0u};
      if (g == 0) p.lse[(int64_t)b * p.heads + h] = -__builtin_inff();
    } else {
      uint16_t* o = p.part16 + ((int64_t)split_slot * p.heads + h) * 512 + 4 * g;
#pragma unroll
      for (int k = 0; k < 64; ++k) *reinterpret_cast<u32x2*>(o + 8 * k) = u32x2{0u, 0u};
      if (g == 0) p.part_lse[(int64_t)split_slot * p.heads + h] = -__builtin_inff();   // low bit 0: fp16 row
    }
    return;
  }

  // Queries.  A wave's 32 heads x 576 values have the shape of a cache tile
  // (32 rows of 512 latent + 64 RoPE values), so the wave loads them like
  // one, into ring slot `wave` with the tile's layout and swizzle: every load
  // moves one whole 1 KiB row (or the RoPE parts of 8 rows), where loading
  // each lane's operand straight from memory would touch 32 rows per load.
  // The score MFMA's B operand (head hl, k-step s, half g) then sits exactly
  // where its A operand would for cache row hl, so the K-read addresses give
  // it.  The 32 latent k-steps stay in VGPRs for the whole work item; the 4
  // RoPE k-steps go to this wave's LDS slots (16 bytes per lane,
  // [step][wave][lane]).  Heads past the last compute with a zero query.  The
  // barrier keeps the tile loads out of the ring until every wave has read
  // its queries.
  if (h0 < p.heads) {
    DmaCursor qc{};
    qc.lat_rb = (uint32_t)(p.q_nope_sh * 2);
    qc.rope_rb = (uint32_t)(p.q_pe_sh * 2);
    DmaTile qd;
    qd.lat = reinterpret_cast<const char*>(p.q_nope + (int64_t)b * p.q_nope_sb + (int64_t)h0 * p.q_nope_sh);
    qd.rope = reinterpret_cast<const char*>(p.q_pe + (int64_t)b * p.q_pe_sb + (int64_t)h0 * p.q_pe_sh);
    qd.nlast = min(31, p.heads - 1 - h0);
    qd.lds = lds_u32(lds + wave * kTileBytes);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int part = 0; part < kLoadsPerTile; ++part) issue_part(qc, qd, w, lane16, part);
    }
    wait_cnt<0, 15>();
    const uint32_t base = qd.lds;
#pragma unroll
    for (int st = 0; st < 36; ++st) {
      u32x4 v = st < 32 ? lds_get16(lds_at(xor_add(base, 32u * (st & 7), klx)), 256 * (st >> 3))
                        : lds_get16(lds_at(xor_add(base, 32u * (st - 32), rkx)), 0);
      v = head_ok ? v : u32x4{0u, 0u, 0u, 0u};
      if (st < kQRegSteps) qreg[st < kQRegSteps ? st : 0] = v;
      else *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(qlds + (((st - kQRegSteps) * 4 + wave) * 64 + lane) * 16) = v;
    }
  }
  __syncthreads();

  // FP8 cache: this wave's loads of tile t into its staging slot, and the
  // pieces of widening a staged tile into its ring slot (see issue_part8 and
  // lat8_lane): w8_read fetches staged group u (0..3 latent, 4 RoPE), w8_half
  // widens half h of chunk c (c = 2u + e for latent, 8 for RoPE) and with
  // h = 1 writes the chunk.  Two latent groups are held at a time.
  u32x4 cx[2], cw;
  u32x2 cy;
  auto load8 = [&](int t, int pg) __attribute__((always_inline)) {
    const DmaTile d = cursor_tile<PAGED>(cur, pg, r1, stage8(t));
#pragma unroll
    for (int part = 0; part < kLoadsPerTile8; ++part) issue_part8(cur, d, wave, lane16, part);
    cursor_next<PAGED>(cur, r1);
  };
  auto w8_read = [&](const lds_char* src, int u) __attribute__((always_inline)) {
    if (u < 4) cx[u & 1] = lds_get16(src, 4096 * wave + 1024 * u + (int)lane16);
    else cy = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(src + kLat8Bytes + 512 * wave + 8 * lane);
  };
  auto w8_half = [&](const lds_char* dst, int c, int h) __attribute__((always_inline)) {
    const uint32_t a = c < 8 ? cx[(c >> 1) & 1][2 * (c & 1) + h] : (h ? cy.y : cy.x);
    cw[2 * h] = widen2<DT, false>(a);
    cw[2 * h + 1] = widen2<DT, true>(a);
    if (h == 1) {
      const uint32_t addr =
          c < 8 ? xor_add(lds_u32(dst) + 8192u * wave + 2048u * (c >> 1), lat8_key(wave, c >> 1, c & 1), lat8_lane(lane))
                : xor_add(lds_u32(dst) + kLatBytes + 1024u * wave, 64u * (wave & 1), rope8_lane(lane));
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>((lds_char*)(uintptr_t)addr) = cw;
    }
  };
  // A whole staged tile at once (prologue, idle waves).
  auto widen_all = [&](const lds_char* src, const lds_char* dst) __attribute__((always_inline)) {
    w8_read(src, 0);
    w8_read(src, 1);
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      w8_half(dst, c, 0);
      w8_half(dst, c, 1);
      if (c == 1) w8_read(src, 2);
      if (c == 3) w8_read(src, 3);
      if (c == 5) w8_read(src, 4);
    }
  };
  // FP8 prologue: tiles 0 and 1 staged and widened into ring slots 0 and 1,
  // tiles 2 and 3 in flight into the staging slots (each issued once its
  // slot's bytes have been widened); every wave's widening done at the
  // barrier.
  auto prologue8 = [&]() __attribute__((always_inline)) {
    load8(0, PAGED ? cursor_page(cur) : 0);
    load8(1, PAGED ? cursor_page(cur) : 0);
    wait_cnt<kLoadsPerTile8, 15>();
    widen_all(stage8(0), slot(0));
    load8(2, PAGED ? cursor_page(cur) : 0);
    wait_cnt<kLoadsPerTile8, 15>();
    widen_all(stage8(1), slot(1));
    load8(3, PAGED ? cursor_page(cur) : 0);
    wait_cnt<63, 0>();
    barrier();
  };

  // A wave whose 32 heads all lie past the last head (few heads per group)
  // computes nothing: it only issues its share of every tile's loads (and
  // with an FP8 cache widens what it loaded) and passes the same barriers as
  // the other waves (prologue; one per step; the one before the epilogue),
  // then leaves.  Wave 0 always has heads.
  if (h0 >= p.heads) {
    if constexpr (KV8) {
      prologue8();
    } else {
#pragma unroll
      for (int kk = 0; kk < 3; ++kk) {
        const int pg = PAGED ? cursor_page(cur) : 0;
        const DmaTile d = cursor_tile<PAGED>(cur, pg, r1, slot(kk));
#pragma unroll
        for (int part = 0; part < kLoadsPerTile; ++part) issue_part(cur, d, wave, lane16, part);
        cursor_next<PAGED>(cur, r1);
      }
      wait_cnt<2 * kLoadsPerTile, 15>();
      barrier();
    }
    int pg_next = 0;
    if (n_tiles > 1) {
      if constexpr (PAGED) pg_next = cursor_page(cur);
      if constexpr (KV8) wait_cnt<63, 0>();
      else wait_cnt<kLoadsPerTile, 0>();
      barrier();
    }
    for (int t = 1; t < n_tiles; ++t) {
      if constexpr (KV8) {
        // step t: tile t+1 widened, tile t+3 loaded into its staging slot
        wait_cnt<kLoadsPerTile8, 15>();
        widen_all(stage8(t + 1), slot(t + 1));
        load8(t + 3, pg_next);
        if constexpr (PAGED) pg_next = cursor_page(cur);
        wait_cnt<63, 0>();
      } else {
        const DmaTile d = cursor_tile<PAGED>(cur, pg_next, r1, slot(t + 2));
        cursor_next<PAGED>(cur, r1);
#pragma unroll
        for (int part = 0; part < kLoadsPerTile; ++part) issue_part(cur, d, wave, lane16, part);
        if constexpr (PAGED) pg_next = cursor_page(cur);
        wait_cnt<kLoadsPerTile, 0>();
      }
      barrier();
    }
    wait_cnt<0, 15>();
    __syncthreads();   // the computing waves' barrier before their epilogue
    return;
  }

  f32x16 acc[16];
#pragma unroll
  for (int vb = 0; vb < 16; ++vb) acc[vb] = f32x16{};
  // nmc = -c m for the reference max m, set from the first tile (Softmax).
  float nmc = 0.f;
  float lsum = 0.f;   // this lane's share of the sum of P (fp32 values)
  float lsr = 0.f;    // fp16: the same of the rounded values

  {
    // ---- prologue ----------------------------------------------------------
    // Always three tiles (FP8: four; the last one again past the end), so
    // that every wait below counts the same loads.
    if constexpr (KV8) {
      prologue8();
    } else {
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int pg = PAGED ? cursor_page(cur) : 0;
        const DmaTile d = cursor_tile<PAGED>(cur, pg, r1, slot(k));
#pragma unroll
        for (int part = 0; part < kLoadsPerTile; ++part) issue_part(cur, d, wave, lane16, part);
        cursor_next<PAGED>(cur, r1);
      }
      wait_cnt<2 * kLoadsPerTile, 15>();
      barrier();
    }

    // LDS operands are read kKA (score) / kVA (value) MFMAs ahead, as far as
    // the registers allow: value operands three ahead for fp16, two for bf16
    // (whose split P takes the registers).  Ring sizes: read-ahead + the
    // operand in use (an MFMA has taken its A and B operands once it issues).
    constexpr int kKA = 2;
    constexpr int kVA = DT == MLA_DTYPE_F16 ? 3 : 2;
    constexpr int kKB = kKA + 1, kVB = kVA + 1;
    u32x4 kb[kKB], vbuf[kVB], qb[4];
    uint32_t kq[8], vw[4], vw1[4];
    f32x16 sA, sB;
    Softmax<DT> sm;

    // Score-operand bases of a tile, then its first kKA K reads.
    auto k_head = [&](const lds_char* tile) __attribute__((always_inline)) {
      const uint32_t base = lds_u32(tile);
#pragma unroll
      for (int j = 0; j < 8; ++j) kq[j] = xor_add(base, 32u * j, klx);
#pragma unroll
      for (int s = 0; s < kKA; ++s) kb[s] = lds_get16(lds_at(kq[s]), 0);
    };
    auto k_read = [&](const lds_char* tile, int s) __attribute__((always_inline)) -> u32x4 {
      if (s < 32) return lds_get16(lds_at(kq[s & 7]), 256 * (s >> 3));
      return lds_get16(lds_at(xor_add(lds_u32(tile), 32u * (s - 32), rkx)), 0);
    };
    // B operand of score step s: Q in VGPRs, or the RoPE part read from LDS.
    auto q_op = [&](int s) __attribute__((always_inline)) -> const u32x4& {
      return s < kQRegSteps ? qreg[s < kQRegSteps ? s : 0] : qb[s < kQRegSteps ? 0 : s - kQRegSteps];
    };
    // Value-operand bases of a tile; operand i = 2 vb + kt, two reads: half r
    // = 1 is half 0 with bit 5 flipped (vofs1 above), kept in registers of
    // its own (forming it at each read cost one VALU op per operand).
    auto v_bases = [&](const lds_char* tile) __attribute__((always_inline)) {
      const uint32_t base = lds_u32(tile);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        vw[cc] = xor_add(base, 64u * cc, vofs0);
        vw1[cc] = xor_add(base, 64u * cc + 32u, vofs0);
      }
    };
    auto v_read = [&](int i) __attribute__((always_inline)) -> u32x4 {
      const int vb = i >> 1, kt = i & 1;
      const int imm = 256 * (vb >> 2) + 16384 * kt;
      return lds_get_tr(lds_at(vw[vb & 3]), imm, lds_at(vw1[vb & 3]), imm + 8192);
    };
    // A tile whose max passed the reference by more than the margin (Softmax
    // step 5 leaves dn < -margin): raise the reference to that max and scale
    // the accumulator and the running sums by alpha = 2^dn, before this
    // tile's exponentials.  The accumulator then holds the tiles before it;
    // their last P·V MFMAs are complete (the padding waits them out anyway).
    // Rare (never on N(0,1) inputs), so a wave-uniform branch: scaling the
    // 256 AGPRs takes some 800 instructions.  One asm statement per register
    // (read, multiply, write back): a vector multiply of the accumulator
    // tiles lets the register allocator move them to VGPRs and spill the
    // queries inside the tile loop.
    auto rescale = [&]() __attribute__((always_inline)) {
      if (__builtin_amdgcn_ballot_w64(sm.dn < -kRescaleMargin<DT>) != 0) {
        const float dz = sm.dn < -kRescaleMargin<DT> ? sm.dn : 0.f;
        const float alpha = __builtin_amdgcn_exp2f(dz);
        nmc += dz;
        lsum *= alpha;
        lsr *= alpha;
        nops_after_mfma(acc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            float tmp;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(acc[i][j]), "=&v"(tmp)
                         : "v"(alpha));
          }
        }
        nops_after_mfma(acc);
      }
    };

    // Score MFMAs of one tile into `sc`; with WITH_SM, the softmax of the
    // previous tile runs between them and the first kVA V reads of the
    // previous tile are issued at the end.
    auto phase_a = [&](const lds_char* tile, f32x16& sc, f32x16& prev, bool with_sm, bool first_prev,
                       const lds_char* vtile) __attribute__((always_inline)) {
      if (with_sm) {
        // Tile 0's scores come straight from its MFMAs: pad the hazard.
        if (first_prev) nops_after_mfma(prev);
#pragma unroll
        for (int e = 0; e < 16; ++e) sm.x[e] = prev[e];
      }
      auto a_step = [&](int s) __attribute__((always_inline)) {
        if (s == 0) mfma_v<DT, true>(sc, kb[0], qreg[0]);
        else mfma_v<DT, false>(sc, kb[s % kKB], q_op(s));
        if (s + kKA < 36) kb[(s + kKA) % kKB] = k_read(tile, s + kKA);
        if (s + kKA >= kQRegSteps && s + kKA < 36)
          qb[s + kKA - kQRegSteps] = lds_get16(lds_at(xor_add(qwave, 0u, lane16)), (s + kKA - kQRegSteps) * 4096);
        if (with_sm) {
          if (s < kSoftmaxSteps<DT>) sm.step(s, first_prev, c, nmc, lsum, lsr);
          if (s == 30) v_bases(vtile);
          if (s >= 36 - kVA) vbuf[s - (36 - kVA)] = v_read(s - (36 - kVA));
        }
        fence();
      };
      // The rescale branch sits between softmax steps 5 and 6, outside the
      // unrolled loops (inside one, it stops the unrolling).
#pragma unroll
      for (int s = 0; s < 6; ++s) a_step(s);
      if (with_sm) {
        rescale();
        fence();
      }
#pragma unroll
      for (int s = 6; s < 36; ++s) a_step(s);
    };
    // P·V MFMAs of one tile, operands [i0, i1), V reads kVA ahead.  With
    // WITH_DMA, this wave's 9 loads of tile dma_t (page dma_pg) go one every
    // three MFMAs: the CU's vector-memory path takes a 1 KiB load only every
    // dozen or so cycles, and a wave stalls at issue until its load is taken
    // (about 20 cycles alone, about 50 when all four waves issue together),
    // so loads issued in a burst stall the MFMAs behind them.  (Loads placed
    // between the score MFMAs, whose accumulator is in VGPRs, stalled longer
    // still.)
    // FP8 cache: WITH_DMA also widens tile w_t (staged, into its ring slot)
    // between the MFMAs, half a chunk per MFMA, each staged group read a few
    // MFMAs ahead; after MFMA 0 the wave waits for its own loads of that
    // tile (those of the next tile may still be in flight).  The 6 loads of
    // tile dma_t go into the staging slot just widened, each once the group
    // it overwrites has been read (its chunks written).
    auto pv_range = [&](int i0, int i1, bool with_dma, int dma_t, int dma_pg, int w_t) __attribute__((always_inline)) {
      DmaTile dt{};
      if (i0 == 0 && with_dma) {
        dt = cursor_tile<PAGED>(cur, dma_pg, r1, KV8 ? stage8(dma_t) : slot(dma_t));
        cursor_next<PAGED>(cur, r1);
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i >= i0 && i < i1) {
          mfma_a<DT>(acc[i >> 1], vbuf[i % kVB], sm.pk[i & 1]);
          if (i0 == 0 && with_dma) {
            if constexpr (KV8) {
              const lds_char* src = stage8(w_t);
              const lds_char* dst = slot(w_t);
              if (i == 0) {
                wait_cnt<kLoadsPerTile8, 15>();
                w8_read(src, 0);
                w8_read(src, 1);
              }
              if (i >= 2 && i < 20) w8_half(dst, (i - 2) >> 1, i & 1);
              if (i == 5) w8_read(src, 2);
              if (i == 9) w8_read(src, 3);
              if (i == 13) w8_read(src, 4);
              // loads: part 0 after group 0 is written (i = 5), ... part 4, 5 after the RoPE (i = 19)
              constexpr int kAt[kLoadsPerTile8] = {7, 11, 15, 17, 19, 21};
#pragma unroll
              for (int q = 0; q < kLoadsPerTile8; ++q)
                if (i == kAt[q]) issue_part8(cur, dt, wave, lane16, q);
            } else if (i % 3 == 1 && i / 3 < kLoadsPerTile) {
              // A load right behind an MFMA, its issue stall overlapping the MFMA.
              issue_part(cur, dt, wave, lane16, i / 3);
            }
          }
          if constexpr (DT == MLA_DTYPE_BF16) mfma_a<DT>(acc[i >> 1], vbuf[i % kVB], sm.pl[i & 1]);
          if (i + kVA < 32) vbuf[(i + kVA) % kVB] = v_read(i + kVA);
          fence();
        }
      }
    };
    // Wait for tile t+1 and for every wave to finish reading tile t-1 (whose
    // slot tile t+3 reuses), then start the K reads of tile t+1.  Returns the
    // page of tile t+3 (paged), loaded before the wait so that the wait
    // covers it.  Uniform: every wave takes the same path.
    auto advance = [&](int t) __attribute__((always_inline)) -> int {
      int pg = 0;
      if constexpr (PAGED) pg = cursor_page(cur);   // the cursor is at tile t+3 (or the last)
      // FP8: tile t+1 was widened in this step (its loads waited for there);
      // the LDS counter covers the widened chunks.
      if constexpr (KV8) wait_cnt<63, 0>();
      else wait_cnt<kLoadsPerTile, 0>();
      barrier();
      k_head(slot(t + 1));
      fence();
      return pg;
    };

    // ---- step 0: scores of tile 0 ------------------------------------------
    k_head(slot(0));
    fence();
    phase_a(slot(0), sA, sB, false, false, slot(0));
    int pg_next = 0;   // page of the tile whose loads the next step issues
    if (n_tiles > 1) pg_next = advance(0);

    // ---- steps 1 .. n-1, two per trip so the score tiles alternate ---------
    // Step t issues tile t+2 into the slot of tile t-2.
    // Every step loads a tile and passes a barrier, also the last ones (see
    // cursor_next), so that the loop has no branch but its back edge.  (Step
    // 1, the softmax of tile 0 that fixes the reference max, stays in the
    // loop: run before it, it made the register allocator move accumulator
    // tiles between the two copies of the step.)
    auto step = [&](int t, f32x16& cur, f32x16& prev) __attribute__((always_inline)) {
      phase_a(slot(t), cur, prev, true, t == 1, slot(t - 1));
      nops_before_mfma<DT>(sm.pk, sm.pl);
      pv_range(0, 32 - kVA, true, KV8 ? t + 3 : t + 2, pg_next, t + 1);
      pg_next = advance(t);
      pv_range(32 - kVA, 32, false, 0, 0, 0);
    };
    // The padding at the end of a trip: with the rescale branch in the loop,
    // the register allocator may swap accumulator tiles on the loop's exit
    // edge, right behind the last P·V MFMA; the wait states cost nothing
    // while that MFMA still occupies the matrix core.
    int t = 1;
    for (; t + 1 < n_tiles; t += 2) {
      step(t, sB, sA);
      step(t + 1, sA, sB);
      nops_after_mfma(acc);
    }
    if (t < n_tiles) step(t, sB, sA);

    // ---- drain: softmax of tile n-1 with the tail masked, its P·V ----------
    // Score tile k was formed in sA for even k, in sB for odd k.
    f32x16 last = ((n_tiles - 1) & 1) ? sB : sA;
    nops_after_mfma(last);
    {
      const int tile_base = r0 + (n_tiles - 1) * kTileRows;
      // This lane's row limit: r1, and in a tail split also the rows its
      // query token t sees (tail_lim + t; tail_lim is INT32_MAX elsewhere).
      const int tok = min(h0 + (lane_id() & 31), p.heads - 1) / p.heads_per_token;
      const int lim = min(r1, tail_lim == INT32_MAX ? INT32_MAX : tail_lim + tok);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int n = 8 * (e >> 2) + 4 * (lane_id() >> 5) + (e & 3);
        sm.x[e] = tile_base + n < lim ? last[e] : -__builtin_inff();
      }
#pragma unroll
      for (int s = 0; s < kSoftmaxSteps<DT>; ++s) {
        sm.step(s, n_tiles == 1, c, nmc, lsum, lsr);
        if (s == 5) rescale();
      }
      v_bases(slot(n_tiles - 1));
#pragma unroll
      for (int i = 0; i < kVA; ++i) vbuf[i] = v_read(i);
      nops_before_mfma<DT>(sm.pk, sm.pl);
      fence();
      pv_range(0, 32, false, 0, 0, 0);
    }
    // No load may still be writing the ring when the ending reuses it or the
    // workgroup leaves.
    wait_cnt<0, 15>();
    nops_after_mfma(acc);
  }
  // Lane, head and half again, from the lane id rather than the workitem id,
  // so that none of them stays live through the tile loop.
  const int lane_t = lane_id();
  const int g_t = lane_t >> 5;
  const int h_t = h0 + (lane_t & 31);
  const bool head_ok_t = h_t < p.heads;
  // ---- epilogue: normalise; write final output or the split partial --------
  // lse from the fp32 sum; the output normalised by the sum of the values the
  // P·V product used (fp16: the rounded sum; see Softmax).
  const float ltot = halves_sum(lsum);
  const float lnorm = DT == MLA_DTYPE_F16 ? halves_sum(lsr) : ltot;
  const bool nonempty = ltot > 0.f;
  // FP8 cache: the products used the stored values; the scale multiplies
  // the normalised output (and is already in c for the scores).
  const float inv = nonempty ? (KV8 ? p.out_scale : 1.f) / lnorm : 0.f;
  const float lse2 = nonempty ? __log2f(ltot) - nmc : -__builtin_inff();
  if (s_b == 1 && head_ok_t && g_t == 0) p.lse[(int64_t)b * p.heads + h_t] = nonempty ? lse2 * kLn2 : -__builtin_inff();
  // The rows leave through LDS: each wave stages its 32 head rows in a
  // region of its own, then writes one whole row (1 KiB, 16 bytes per lane)
  // per store instruction.  Straight from the accumulator layout, a store
  // would cover 16-byte pieces of 32 rows.  Staged 16-byte chunk c of row r
  // sits at chunk c ^ r: the accumulator writes (32 rows) and the row reads
  // (64 chunks of one row) are both free of bank conflicts.  The barrier
  // makes sure that every wave has finished reading the tile ring (idle
  // waves pass it too).
  __syncthreads();
  lds_char* stage = lds + wave * 32768;
  const int hl_t = lane_t & 31;
  auto stage_at = [&](int row, int chunk) __attribute__((always_inline)) {
    return stage + row * 1024 + ((chunk ^ row) << 4);
  };
  // 16-bit rows, 512 values = 64 chunks of 8; this lane holds values
  // 8 q + 4 g .. + 3 of chunk 4 vb + q.  ODT: the output's type, or fp16 for
  // a partial, whose largest |value| (this lane's half row) it returns.
  auto stage16 = [&](auto odt, auto partial) __attribute__((always_inline)) -> float {
    constexpr int ODT = decltype(odt)::value;
    constexpr bool PART = decltype(partial)::value;
    float rmax = 0.f;
#pragma unroll
    for (int vb = 0; vb < 16; ++vb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a0 = acc[vb][4 * q + 0] * inv, a1 = acc[vb][4 * q + 1] * inv;
        const float a2 = acc[vb][4 * q + 2] * inv, a3 = acc[vb][4 * q + 3] * inv;
        if (PART) {
          rmax = max3_abs(rmax, a0, a1);
          rmax = max3_abs(rmax, a2, a3);
        }
        u32x2 w;
        w.x = pack2<ODT>(a0, a1);
        w.y = pack2<ODT>(a2, a3);
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(stage_at(hl_t, 4 * vb + q) + 8 * g_t) = w;
      }
    }
    return rmax;
  };
  // skip_rows: bit r set leaves row r out (a partial row kept in fp32).
  auto store16 = [&](uint16_t* row0, int64_t row_stride, uint32_t skip_rows) __attribute__((always_inline)) {
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
      if (h0 + r >= p.heads) break;
      if ((skip_rows >> r) & 1u) continue;
      const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(stage_at(r, lane_t));
      *reinterpret_cast<u32x4*>(row0 + r * row_stride + 8 * lane_t) = v;
    }
  };
  if (s_b == 1) {
    stage16(std::integral_constant<int, DT>{}, std::false_type{});
    store16(p.out + (int64_t)b * p.out_sb + (int64_t)h0 * p.out_sh, p.out_sh, 0u);
    return;
  }
  // Split partial.  A row whose values all lie within +-kPart16Max goes out
  // in fp16; a wider one in fp32 only (its fp16 slot is left as it was), and
  // the low bit of its lse says so.  An fp16 row then adds at most 2^-12
  // (half an ulp below 1) per value to the combined output, whatever the
  // weights; a 16-bit copy of larger values would add 2^-12 |O_k|, which
  // exceeds the absolute tolerance where large value rows of two splits
  // cancel.
  const float rmax = halves_max(stage16(std::integral_constant<int, MLA_DTYPE_F16>{}, std::true_type{}));
  const bool big = rmax > kPart16Max;
  if (head_ok_t && g_t == 0)
    p.part_lse[(int64_t)split_slot * p.heads + h_t] = lse_with_flag(lse2, big);
  const uint32_t bigrows = (uint32_t)__builtin_amdgcn_ballot_w64(big);   // bit r: head h0 + r
  store16(p.part16 + ((int64_t)split_slot * p.heads + h0) * 512, 512, bigrows);
  if (bigrows == 0) return;
  // fp32 rows of the large ones, in two halves of 256 values = 64 chunks of
  // 4; this lane holds chunk 8 (vb % 8) + 2 q + g.  The products are formed
  // again from the accumulator (an opaque copy of inv keeps the compiler from
  // holding the fp16 path's products, 256 registers, until here).
  float inv32 = inv;
  asm volatile("" : "+v"(inv32));
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int vb = 8 * half; vb < 8 * half + 8; ++vb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 w = {acc[vb][4 * q + 0] * inv32, acc[vb][4 * q + 1] * inv32, acc[vb][4 * q + 2] * inv32,
                         acc[vb][4 * q + 3] * inv32};
        *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(stage_at(hl_t, 8 * (vb & 7) + 2 * q + g_t)) = w;
      }
    }
    for (int r = 0; r < 32; ++r) {
      if (h0 + r >= p.heads) break;
      if (((bigrows >> r) & 1u) == 0) continue;
      float* row = p.part32 + ((int64_t)split_slot * p.heads + h0 + r) * 512 + 256 * half;
      const f32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(stage_at(r, lane_t));
      *reinterpret_cast<f32x4*>(row + 4 * lane_t) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Combine kernels.  combine_heads_kernel: grid (ceil(H / 4), B), one wave per
// head, 8 output values per lane; for sequences of few splits.
// combine_splitk_kernel: grid (H, B), four waves per head; for many splits,
// where one wave per head would leave most of the GPU idle.  Both form the
// final LSE from all split lse values first, then the weighted sum.
// ---------------------------------------------------------------------------

// Float max / sum over a wave: DPP within each row of 16 lanes, then the four
// row results read out (the result is wave-uniform).
template <int CTRL>
__device__ __forceinline__ float mov_dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, mov_dpp_f32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, mov_dpp_f32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, mov_dpp_f32<0x141>(v));   // row_half_mirror
  v = fmaxf(v, mov_dpp_f32<0x140>(v));   // row_mirror
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += mov_dpp_f32<0xB1>(v);
  v += mov_dpp_f32<0x4E>(v);
  v += mov_dpp_f32<0x141>(v);
  v += mov_dpp_f32<0x140>(v);
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}

// Eight values (element offset e) of a partial row: fp16 rows in one 16-byte
// read (kept as read until they are added, half the registers of fp32),
// fp32 rows in two.
__device__ __forceinline__ u32x4 load_part16x8(const uint16_t* part16, int64_t e) {
  return *reinterpret_cast<const u32x4*>(part16 + e);
}
__device__ __forceinline__ void load_part32x8(const float* part32, int64_t e, f32x4& v0, f32x4& v1) {
  const f32x4* src = reinterpret_cast<const f32x4*>(part32 + e);
  v0 = src[0];
  v1 = src[1];
}

// a += w v for an fp16 partial row (8 values as read), or nothing when
// `skip`: a wide split, whose fp16 slot holds stale bits (possibly NaN), or a
// batch entry past the last split, which re-read the last one (possibly
// wide).  The product is selected away rather than weighted by 0, since
// 0 * NaN is NaN.
__device__ __forceinline__ void add_fp16_part(f32x4& a0, f32x4& a1, float w, u32x4 raw, bool skip) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const f32x4 v0 = __builtin_convertvector(__builtin_bit_cast(h4, u32x2{raw.x, raw.y}), f32x4);
  const f32x4 v1 = __builtin_convertvector(__builtin_bit_cast(h4, u32x2{raw.z, raw.w}), f32x4);
  const f32x4 t0 = w * v0, t1 = w * v1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a0[i] += skip ? 0.f : t0[i];
    a1[i] += skip ? 0.f : t1[i];
  }
}

// a += w(u) v_u for the wide splits u of a batch of U (bit u of `wide`):
// their fp32 rows at O + first + u * step, read four at a time, each four
// before any is added; the other slots of a four re-read the batch's first
// wide row (a cache hit) and add it with weight 0.
template <int U, typename WeightOf>
__device__ __forceinline__ void add_fp32_parts(f32x4& a0, f32x4& a1, const float* part32, int64_t O, int64_t step,
                                               int64_t first, uint32_t wide, WeightOf weight_of) {
  if (wide == 0) return;
  const int f = __builtin_ctz(wide);
  constexpr int G = U < 4 ? U : 4;
#pragma unroll
  for (int u0 = 0; u0 < U; u0 += G) {
    if (((wide >> u0) & ((1u << G) - 1u)) == 0) continue;
    f32x4 w0[G], w1[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int u = u0 + g;
      const int uu = ((wide >> u) & 1u) ? u : f;
      load_part32x8(part32, O + first + (int64_t)uu * step, w0[g], w1[g]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float w = ((wide >> (u0 + g)) & 1u) ? weight_of(u0 + g) : 0.f;
      a0 += w * w0[g];
      a1 += w * w1[g];
    }
  }
}

constexpr int kCombineUnroll = 8;   // splits per wave whose reads are in flight together (one wave per head)
constexpr int kSplitkBatch = 16;    // the same for each of the four waves of a head

// Number of splits of sequence b and its first work item.
__device__ __forceinline__ void combine_range(const CombineParams& p, int b, int& s, int& base) {
  if (p.num_split > 0) {
    s = p.num_split;
    base = b * p.num_split;
  } else {
    base = min(max(p.split_offset[b], 0), p.max_work);
    s = min(max(p.split_offset[b + 1], base), p.max_work) - base;
  }
}

// Final base-2 lse of a head from the split lse values held two per lane
// (l0 of split lane, l1 of split lane + 64; -inf past the splits; format
// bits already cleared) plus any splits beyond the first 128, and this lane's
// weight for split `lane`.  A head whose splits are all empty gets total =
// -inf and weight 0 everywhere (output 0, lse -inf), without a branch, so
// that the partial-row reads already in flight stay in flight.
struct CombineWeights {
  float total, w_own;
};
__device__ __forceinline__ CombineWeights combine_weights(float l0, float l1, const float* L, int heads, int s,
                                                          int lane) {
  float mx = fmaxf(l0, l1);
  for (int k = lane + 128; k < s; k += 64) mx = fmaxf(mx, lse_value(L[(int64_t)k * heads]));
  mx = wave_max(mx);
  const float ref = mx == -__builtin_inff() ? 0.f : mx;
  float se = __builtin_amdgcn_exp2f(l0 - ref) + __builtin_amdgcn_exp2f(l1 - ref);   // 0 past s
  for (int k = lane + 128; k < s; k += 64) se += __builtin_amdgcn_exp2f(lse_value(L[(int64_t)k * heads]) - ref);
  se = wave_sum(se);
  const float total = __log2f(se) + ref;   // -inf when every split is empty
  const float w_own = se > 0.f ? __builtin_amdgcn_exp2f(l0 - total) : 0.f;
  return {total, w_own};
}

// lse of split k = lane + 64 j as held by the lane, with its format bit
// (-inf past s), read without a branch: lanes past s re-read split s - 1.
__device__ __forceinline__ float lane_lse(const float* L, int heads, int s, int k) {
  const float l = L[(int64_t)(k < s ? k : s - 1) * heads];
  return k < s ? l : -__builtin_inff();
}

// One wave merges the s splits of head h of sequence b; lane l owns output
// columns 8 l .. 8 l + 7.  S = s when s is 2..kCombineUnroll (every read of
// the partial rows issued before the first wait), S = 0 for any larger count.
// The fp16 rows are read together with the lse values and accumulated; a
// split whose lse carries the format bit (its fp16 slot holds stale data,
// selected away) has its fp32 row read and added afterwards.
template <int DT, int S>
__device__ __forceinline__ void combine_head(const CombineParams& p, int b, int h, int lane, int s_rt, int base) {
  constexpr int U = S ? S : kCombineUnroll;
  const int s = S ? S : s_rt;
  const float* L = p.part_lse + (int64_t)base * p.heads + h;
  const int64_t stride = (int64_t)p.heads * 512;   // elements between consecutive splits
  const int64_t O = ((int64_t)base * p.heads + h) * 512 + 8 * lane;
  // Lane k holds the lse of split k (and k + 64).  The first U partial rows
  // are read in the same round trip: they do not depend on the weights.
  const float r0 = lane_lse(L, p.heads, s, lane);
  const float r1 = S ? -__builtin_inff() : lane_lse(L, p.heads, s, lane + 64);
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = load_part16x8(p.part16, O + (int64_t)u * stride);
  __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the reductions
  const uint64_t wide = __builtin_amdgcn_ballot_w64(lse_flag(r0));   // bit k: split k has an fp32 row
  const CombineWeights cw = combine_weights(lse_value(r0), lse_value(r1), L, p.heads, s, lane);
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float w = lane_f32(cw.w_own, u);   // split u's weight, held by lane u
    add_fp16_part(a0, a1, w, v[u], (wide >> u) & 1ull);
  }
  add_fp32_parts<U>(a0, a1, p.part32, O, stride, 0, (uint32_t)(wide & ((1ull << U) - 1ull)),
                    [&](int u) __attribute__((always_inline)) { return lane_f32(cw.w_own, u); });
  if constexpr (S == 0) {
    // s > U: further batches of U; indices past s re-read split s - 1 with weight 0.
    const bool any = cw.total != -__builtin_inff();
    for (int k0 = U; k0 < s; k0 += U) {
      float lk[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + u < s ? k0 + u : s - 1;
        v[u] = load_part16x8(p.part16, O + (int64_t)k * stride);
        lk[u] = L[(int64_t)k * p.heads];
      }
      auto weight_of = [&](int u) __attribute__((always_inline)) {
        return any && k0 + u < s ? __builtin_amdgcn_exp2f(lse_value(lk[u]) - cw.total) : 0.f;
      };
      uint32_t wm = 0;   // lk[u] is the same in every lane
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool wd = k0 + u < s && lse_flag(lk[u]);
        wm |= wd ? 1u << u : 0u;
        add_fp16_part(a0, a1, weight_of(u), v[u], wd || k0 + u >= s);
      }
      add_fp32_parts<U>(a0, a1, p.part32, O, stride, (int64_t)k0 * stride, wm, weight_of);
    }
  }
  u32x4 r;
  r.x = pack2<DT>(a0.x, a0.y);
  r.y = pack2<DT>(a0.z, a0.w);
  r.z = pack2<DT>(a1.x, a1.y);
  r.w = pack2<DT>(a1.z, a1.w);
  uint16_t* o = p.out + (int64_t)b * p.out_sb + (int64_t)h * p.out_sh + 8 * lane;
  *reinterpret_cast<u32x4*>(o) = r;
  if (lane == 0) p.lse[(int64_t)b * p.heads + h] = cw.total * kLn2;
}

// Grid position (x, y) of this workgroup, remapped so that each XCD runs a
// contiguous run of (x, y) in y-major order.  The split kernel gives each XCD
// a contiguous run of work items, i.e. of sequences, so a sequence's partials
// are then read on the XCD whose L2 took their writes.  A bijection of the
// grid (the dispatcher deals flat ids to the XCDs round-robin).
__device__ __forceinline__ void xcd_grid_pos(int& x, int& y) {
  const int total = gridDim.x * gridDim.y;
  const int flat = blockIdx.x + blockIdx.y * gridDim.x;
  const int xcd = flat & (kXcds - 1), idx = flat / kXcds;
  const int lin = xcd * (total / kXcds) + min(xcd, total % kXcds) + idx;
  y = lin / gridDim.x;
  x = lin - y * gridDim.x;
}

template <int DT>
__global__ __launch_bounds__(256) void combine_heads_kernel(CombineParams p) {
  int hx, b;
  xcd_grid_pos(hx, b);
  const int h = hx * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (h >= p.heads) return;
  int s, base;
  combine_range(p, b, s, base);
  static_assert(kCombineUnroll == 8, "the cases below list 2..kCombineUnroll");
  switch (s) {
    case 0:
    case 1: return;   // one split wrote out/lse itself
    case 2: combine_head<DT, 2>(p, b, h, lane, s, base); break;
    case 3: combine_head<DT, 3>(p, b, h, lane, s, base); break;
    case 4: combine_head<DT, 4>(p, b, h, lane, s, base); break;
    case 5: combine_head<DT, 5>(p, b, h, lane, s, base); break;
    case 6: combine_head<DT, 6>(p, b, h, lane, s, base); break;
    case 7: combine_head<DT, 7>(p, b, h, lane, s, base); break;
    case 8: combine_head<DT, 8>(p, b, h, lane, s, base); break;
    default: combine_head<DT, 0>(p, b, h, lane, s, base); break;
  }
}

// Wave w accumulates splits w, w + 4, ... in batches of kSplitkBatch (8
// output values per lane), then the four sums meet in LDS and wave w writes
// output columns 128 w .. 128 w + 127.  A batch's lse values are read one
// batch ahead, so that each partial row is read in its own format, fp16 or
// (format bit set) fp32, and a batch costs one memory round trip: its rows
// go out together with the next batch's lse values.
template <int DT>
__global__ __launch_bounds__(256) void combine_splitk_kernel(CombineParams p) {
  __shared__ f32x4 red[4][2][64];   // [wave][half][lane]: 8 values per lane
  int h, b;
  xcd_grid_pos(h, b);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int s, base;
  combine_range(p, b, s, base);
  if (s <= 1) return;   // one split wrote out/lse itself

  constexpr int U = kSplitkBatch;
  const float* L = p.part_lse + (int64_t)base * p.heads + h;
  const int64_t stride = (int64_t)p.heads * 512;   // elements between consecutive splits
  const int64_t O = ((int64_t)base * p.heads + h) * 512 + 8 * lane;
  // Batch of this wave's splits k0, k0 + 4, ..., k0 + 4 (U - 1); indices past
  // s re-read split s - 1 and are left out of the sum.
  float lk[U], lkn[U];   // the batch's lse values (with format bits), the next batch's
  auto load_lse = [&](int k0, float* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + 4 * u < s ? k0 + 4 * u : s - 1;
      dst[u] = L[(int64_t)k * p.heads];
    }
  };
  // Row of split k: 16 bytes of fp16 (va; vb the same again) or 32 bytes of
  // fp32 (va, vb), chosen by its format bit.
  u32x4 va[U], vb[U];
  auto load_rows = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + 4 * u < s ? k0 + 4 * u : s - 1;
      const int64_t e = O + (int64_t)k * stride;
      const u32x4* pa = lse_flag(lk[u]) ? reinterpret_cast<const u32x4*>(p.part32 + e)
                                        : reinterpret_cast<const u32x4*>(p.part16 + e);
      va[u] = pa[0];
      vb[u] = pa[lse_flag(lk[u]) ? 1 : 0];
    }
  };

  load_lse(wave, lk);
  const float l0 = lane_lse(L, p.heads, s, lane), l1 = lane_lse(L, p.heads, s, lane + 64);
  const CombineWeights cw = combine_weights(lse_value(l0), lse_value(l1), L, p.heads, s, lane);
  const bool any = cw.total != -__builtin_inff();

  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = wave;;) {
    load_rows(k0);
    const int kn = k0 + 4 * U;
    if (kn < s) load_lse(kn, lkn);
    __builtin_amdgcn_sched_barrier(0);   // both sets of reads ahead of the sums
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!any || k0 + 4 * u >= s) continue;   // uniform: lk[u] is the same in every lane
      const float w = __builtin_amdgcn_exp2f(lse_value(lk[u]) - cw.total);
      if (lse_flag(lk[u])) {
        a0 += w * __builtin_bit_cast(f32x4, va[u]);
        a1 += w * __builtin_bit_cast(f32x4, vb[u]);
      } else {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        a0 += w * __builtin_convertvector(__builtin_bit_cast(h4, u32x2{va[u].x, va[u].y}), f32x4);
        a1 += w * __builtin_convertvector(__builtin_bit_cast(h4, u32x2{va[u].z, va[u].w}), f32x4);
      }
    }
    k0 = kn;
    if (k0 >= s) break;
#pragma unroll
    for (int u = 0; u < U; ++u) lk[u] = lkn[u];
  }
  red[wave][0][lane] = a0;
  red[wave][1][lane] = a1;
  __syncthreads();
  // Wave w: columns 128 w + 2 lane, + 1 (lane pair 16 w + lane / 4 of the
  // 8-value lanes above, half (lane / 2) % 2, element pair lane % 2).
  const int src_lane = 16 * wave + (lane >> 2), half = (lane >> 1) & 1, e = 2 * (lane & 1);
  float c0 = 0.f, c1 = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const f32x4 q = red[v][half][src_lane];
    c0 += q[e];
    c1 += q[e + 1];
  }
  uint16_t* o = p.out + (int64_t)b * p.out_sb + (int64_t)h * p.out_sh + 128 * wave + 2 * lane;
  *reinterpret_cast<uint32_t*>(o) = pack2<DT>(c0, c1);
  if (wave == 0 && lane == 0) p.lse[(int64_t)b * p.heads + h] = cw.total * kLn2;
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
  const int sq = p.seqlen_q, tail = tail_splits(sq);
  auto pre_blocks = [&](int b) { return num_blocks(prefix_len(clamp_len(p.seqlens[b], p.row_cap), sq)); };
  int t = 1;
  if (p.num_split == 0) {
    int mx = 0;
    for (int b = tid; b < B; b += kPlanThreads) mx = max(mx, pre_blocks(b));
    mx = block_max(mx, red);
    const int cap = planner_cap(B, p.heads, p.num_cus, sq);
    int lo = 1, hi = mx > 1 ? mx : 1;
    while (lo < hi) {
      const int mid = lo + (hi - lo) / 2;
      int cnt = 0;
      for (int b = tid; b < B; b += kPlanThreads) cnt += splits_for_budget(pre_blocks(b), mid);
      cnt = block_sum(cnt, red);
      if (cnt <= cap) hi = mid; else lo = mid + 1;
    }
    t = lo;
  }
  // Prefix splits of sequence b.
  auto spre_of = [&](int b) { return p.num_split > 0 ? p.num_split : splits_for_budget(pre_blocks(b), t); };

  // Contiguous chunk of sequences per thread; exclusive scan of chunk totals.
  const int per = (B + kPlanThreads - 1) / kPlanThreads;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int mine = 0;
  for (int b = b0; b < b1; ++b) mine += spre_of(b) + tail;
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
    const int spre = spre_of(b), s = spre + tail;
    p.num_splits[b] = s;
    p.split_offset[b] = off;
    for (int k = 0; k < s; ++k) {
      int r0, r1;
      seq_split_range(L, sq, spre, k, &r0, &r1);
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
// Block-table check.  The split kernel clamps a page index outside
// [0, num_pages) into the pool: it reads valid memory, but not the rows
// meant.  This kernel (one workgroup per sequence) counts the entries the
// split kernel reads, j < ceil(L_b / page_size) with L_b clamped as there,
// that lie outside the pool: bad[b] for sequence b.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void check_block_table_kernel(BlockCheckParams p) {
  __shared__ int red[256];
  const int b = blockIdx.x;
  const int L = clamp_len(p.seqlens[b], p.row_cap);
  const int nblk = (L + p.page_size - 1) / p.page_size;
  int bad = 0;
  for (int j = threadIdx.x; j < nblk; j += 256) {
    const int pg = p.block_table[(int64_t)b * p.bt_stride + j];
    bad += (pg < 0 || pg >= p.num_pages) ? 1 : 0;
  }
  red[threadIdx.x] = bad;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.bad[b] = red[0];
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// Scratch of the no-allocation entry point (mla_decode_noalloc): a static
// device array, one per GPU the library runs on, held until the process
// ends.  Host code never passes `scratch` itself to a kernel (on the host the
// name is only a stand-in for the device symbol): its device address is taken
// once per device, with that device current, and cached.
// ---------------------------------------------------------------------------

static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* addr[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = MLA_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

hipError_t launch_check_block_table(const BlockCheckParams& p, int batch, hipStream_t stream) {
  hipLaunchKernelGGL(check_block_table_kernel, dim3(batch), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_plan(const PlanParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

// A launch, timed from its dispatch packet when events are given (as a
// profiler times it, without the latency of separate event packets).
template <typename Kernel, typename Params>
static void launch_k(Kernel kernel, dim3 grid, dim3 block, hipStream_t stream, hipEvent_t t0, hipEvent_t t1,
                     const Params& p) {
  if (t0) hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, t0, t1, 0, p);
  else hipLaunchKernelGGL(kernel, grid, block, 0, stream, p);
}

template <int DT, bool KV8>
static void launch_split_dt(const SplitParams& p, bool paged, dim3 grid, hipStream_t stream, hipEvent_t t0,
                            hipEvent_t t1) {
  const bool given = p.num_split == kPlanGiven;
  if (paged) {
    if (given) launch_k(split_kernel<DT, true, KV8, true>, grid, dim3(kThreads), stream, t0, t1, p);
    else launch_k(split_kernel<DT, true, KV8, false>, grid, dim3(kThreads), stream, t0, t1, p);
  } else {
    if (given) launch_k(split_kernel<DT, false, KV8, true>, grid, dim3(kThreads), stream, t0, t1, p);
    else launch_k(split_kernel<DT, false, KV8, false>, grid, dim3(kThreads), stream, t0, t1, p);
  }
}

hipError_t launch_split(const SplitParams& p, int dtype, bool paged, bool kv8, int grid_x, int grid_y,
                        hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const dim3 grid(grid_x, grid_y);
  if (dtype == MLA_DTYPE_F16) {
    if (kv8) launch_split_dt<MLA_DTYPE_F16, true>(p, paged, grid, stream, t0, t1);
    else launch_split_dt<MLA_DTYPE_F16, false>(p, paged, grid, stream, t0, t1);
  } else {
    if (kv8) launch_split_dt<MLA_DTYPE_BF16, true>(p, paged, grid, stream, t0, t1);
    else launch_split_dt<MLA_DTYPE_BF16, false>(p, paged, grid, stream, t0, t1);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int dtype, int batch, int mean_splits, hipStream_t stream,
                          hipEvent_t t0, hipEvent_t t1) {
  const dim3 block(256);
  if (mean_splits >= kCombineSplitkMin) {
    const dim3 grid(p.heads, batch);
    if (dtype == MLA_DTYPE_F16) launch_k(combine_splitk_kernel<MLA_DTYPE_F16>, grid, block, stream, t0, t1, p);
    else launch_k(combine_splitk_kernel<MLA_DTYPE_BF16>, grid, block, stream, t0, t1, p);
  } else {
    const dim3 grid((p.heads + 3) / 4, batch);
    if (dtype == MLA_DTYPE_F16) launch_k(combine_heads_kernel<MLA_DTYPE_F16>, grid, block, stream, t0, t1, p);
    else launch_k(combine_heads_kernel<MLA_DTYPE_BF16>, grid, block, stream, t0, t1, p);
  }
  return hipGetLastError();
}

}  // namespace mla
