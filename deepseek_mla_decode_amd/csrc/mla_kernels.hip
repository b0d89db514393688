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
//     v_mfma_f32_32x32x16: A = 32 cache rows × 16 dims from LDS, B = the wave's
//     Q slice held in 144 VGPRs for the whole work item.  Each lane then holds
//     16 scores of ONE head, so max/sum need a single cross-lane step (lane
//     l ^ 32) and P is already laid out as the B operand of the next product.
//   * Output is also transposed, Oᵀ[v][h] += Vᵀ[v][n]·Pᵀ[n][h]: 16 MFMA tiles
//     of 32 value columns, accumulator 32 heads × 512 fp32 = 256 AGPRs; every
//     value a lane holds belongs to its own head, so rescaling is lane-local.
//   * The KV tile (32 rows) is loaded once per workgroup with 128-bit loads,
//     each wave taking 8 whole rows (one coalesced 1 KiB row per instruction),
//     and written to LDS twice: row-major [32][576] for the score product and,
//     after an 8×8 in-register transpose, value-major [512][32] for P·V.
//     Two LDS buffers of 68 KiB: the next tile's loads are in flight while
//     the current tile is computed.
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
constexpr int kKChunks = (512 + 64) / 8;      // 16-byte chunks per cache row (72)
constexpr int kKBytes = kTileRows * kKChunks * 16;   // 36864
constexpr int kVBytes = 512 * kTileRows * 2;         // 32768
constexpr int kBufBytes = kKBytes + kVBytes;         // 69632
constexpr float kLn2 = 0.69314718055994530942f;
// Lazy rescale threshold (base-2 units): the running max used for the
// exponentials is only raised when a tile's max exceeds it by more than this,
// so unnormalised P stays below 2^8.
constexpr float kRescaleThreshold = 8.0f;

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
// LDS addressing (units of 16-byte chunks inside one buffer)
// ---------------------------------------------------------------------------

// Row-major score operand: row n (0..31), chunk c (0..71; 0..63 latent, 64..71
// RoPE).  XOR of the chunk index with the row's low bits spreads the 8 rows a
// group of 8 lanes reads over all banks.
__device__ __forceinline__ int k_chunk(int n, int c) { return n * kKChunks + (c ^ (n & 7)); }

// Value-major P·V operand: value column v (0..511), chunk c (0..3) of 8
// positions.  Two columns share a 128-byte line; the XOR mask mixes bits of
// v so that both the transposing writes (8 lanes -> columns 8 apart) and the
// MFMA reads (8 lanes -> consecutive columns) hit 8 different 16-byte banks.
__device__ __forceinline__ int v_chunk(int v, int c) {
  const int line = v >> 1;
  const int mask = (line & 3) ^ ((v >> 3) & 7);
  return kKChunks * kTileRows + line * 8 + (((v & 1) * 4 + c) ^ mask);
}

// Position p (0..31) in a value-major column <-> cache row n of the tile.
// The P·V MFMA's contraction slot (half g, element j) of k-step kt carries row
// n = 16kt + 8(j/4) + 4g + (j%4) (the layout in which the score MFMA leaves P);
// storing that row at position p = 16kt + 8g + j makes each lane's operand one
// contiguous 16-byte chunk.  The map swaps bits 2 and 3.
__device__ __forceinline__ int pos_to_row(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

// ---------------------------------------------------------------------------
// Split kernel
// ---------------------------------------------------------------------------

struct TileRegs {
  u32x4 lat[8];   // 8 rows x this lane's 16-byte latent chunk
  u32x4 rope;     // one 16-byte RoPE chunk
};

// Start of the latent (which == 0) or RoPE (which == 1) part of cache row r;
// `sel` is the sequence (contiguous) or the physical page (paged).
template <bool PAGED>
__device__ __forceinline__ const uint16_t* row_ptr(const SplitParams& p, int64_t sel, int r, int which) {
  const int rr = PAGED ? (r % p.page_size) : r;
  if (which == 0) return p.kv + sel * p.kv_sb + (int64_t)rr * p.kv_sr;
  return p.kpe + sel * p.kpe_sb + (int64_t)rr * p.kpe_sr;
}

// Issue the global loads of tile rows [tile_base, tile_base + 32).  Rows at or
// past r1 are redirected to row r1 - 1 (always valid); their scores are masked.
template <bool PAGED>
__device__ __forceinline__ void load_tile(const SplitParams& p, int b, int tile_base, int r1, int wave,
                                          int lane, TileRegs& t) {
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
    int r = tile_base + pos_to_row(8 * wave + i);
    r = r < last ? r : last;
    t.lat[i] = ld16(row_ptr<PAGED>(p, sel, r, 0) + 8 * lane);
  }
  const int tid = wave * 64 + lane;
  int r = tile_base + (tid >> 3);
  r = r < last ? r : last;
  t.rope = ld16(row_ptr<PAGED>(p, sel, r, 1) + 8 * (tid & 7));
}

__device__ __forceinline__ void lds_put(char* base, int byte_off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + byte_off) = v;
}
__device__ __forceinline__ u32x4 lds_get(const char* base, int byte_off) {
  return *reinterpret_cast<const u32x4*>(base + byte_off);
}

// Write a loaded tile into one LDS buffer: row-major copy plus the transposed
// value-major copy.  Offsets are the closed forms of k_chunk / v_chunk for
// the rows and columns this lane owns.
__device__ __forceinline__ void store_tile(char* buf, int wave, int lane, const TileRegs& t) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int n = pos_to_row(8 * wave + i);
    lds_put(buf, 16 * k_chunk(n, lane), t.lat[i]);
  }
  const int tid = wave * 64 + lane;
  lds_put(buf, 16 * k_chunk(tid >> 3, 64 + (tid & 7)), t.rope);
  // 8x8 transpose of 16-bit values: column j of the lane's block (value index
  // 8*lane + j) across its 8 rows (positions 8*wave .. 8*wave + 7).
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    u32x4 ev, od;
    ev.x = __builtin_amdgcn_perm(t.lat[1][q], t.lat[0][q], 0x05040100u);
    ev.y = __builtin_amdgcn_perm(t.lat[3][q], t.lat[2][q], 0x05040100u);
    ev.z = __builtin_amdgcn_perm(t.lat[5][q], t.lat[4][q], 0x05040100u);
    ev.w = __builtin_amdgcn_perm(t.lat[7][q], t.lat[6][q], 0x05040100u);
    od.x = __builtin_amdgcn_perm(t.lat[1][q], t.lat[0][q], 0x07060302u);
    od.y = __builtin_amdgcn_perm(t.lat[3][q], t.lat[2][q], 0x07060302u);
    od.z = __builtin_amdgcn_perm(t.lat[5][q], t.lat[4][q], 0x07060302u);
    od.w = __builtin_amdgcn_perm(t.lat[7][q], t.lat[6][q], 0x07060302u);
    lds_put(buf, 16 * v_chunk(8 * lane + 2 * q, wave), ev);
    lds_put(buf, 16 * v_chunk(8 * lane + 2 * q + 1, wave), od);
  }
}

template <int DT, bool PAGED>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void split_kernel(SplitParams p) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kBufBytes];

  const int wi = blockIdx.x;
  const int hg = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int hl = lane & 31;
  const int g = lane >> 5;

  // ---- work item -----------------------------------------------------------
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

  const int h0 = hg * kHeadsPerGroup + wave * 32;
  const bool wave_active = h0 < p.heads;
  const bool head_ok = h0 + hl < p.heads;
  const int h = head_ok ? h0 + hl : p.heads - 1;   // padded lanes read a valid row, then zero it

  // ---- Q slice: B operand of the score MFMA, k-step s covers dims 16s..16s+15
  u32x4 qreg[36];
  {
    const uint16_t* qn = p.q_nope + (int64_t)b * p.q_nope_sb + (int64_t)h * p.q_nope_sh + 8 * g;
    const uint16_t* qp = p.q_pe + (int64_t)b * p.q_pe_sb + (int64_t)h * p.q_pe_sh + 8 * g;
#pragma unroll
    for (int s = 0; s < 36; ++s) {
      const u32x4 v = s < 32 ? ld16(qn + 16 * s) : ld16(qp + 16 * (s - 32));
      qreg[s] = head_ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x16 acc[16];
#pragma unroll
  for (int vb = 0; vb < 16; ++vb) acc[vb] = f32x16{};
  float m = -__builtin_inff();   // running max used for the exponentials (base 2, scaled)
  float lsum = 0.f;              // this lane's share of the running sum

  // Per-lane LDS byte offsets of the MFMA operands.  Score operand, k-step s:
  // 16*k_chunk(hl, 2s+g) = kofs[s % 4] + 128*(s / 4).  Value operand, column
  // block vb, k-step kt: 16*v_chunk(32vb+hl, 2kt+g) = vofs[kt][vb % 2] + 2048*vb.
  int kofs[4], vofs[2][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) kofs[i] = 16 * k_chunk(hl, 2 * i + g);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    vofs[kt][0] = 16 * v_chunk(hl, 2 * kt + g);
    vofs[kt][1] = 16 * v_chunk(32 + hl, 2 * kt + g) - 2048;
  }

  const int n_tiles = (r1 - r0 + kTileRows - 1) / kTileRows;
  TileRegs tr;
  if (n_tiles > 0) {
    load_tile<PAGED>(p, b, r0, r1, wave, lane, tr);
    store_tile(lds, wave, lane, tr);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int tile_base = r0 + t * kTileRows;
    const bool more = t + 1 < n_tiles;
    if (more) load_tile<PAGED>(p, b, tile_base + kTileRows, r1, wave, lane, tr);

    const char* buf = lds + (t & 1) * kBufBytes;
    if (wave_active) {
      // -- scores: Sᵀ[n][h], n = 8(e/4) + 4g + (e%4) for accumulator element e
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int s = 0; s < 36; ++s) sacc = mfma32<DT>(lds_get(buf + kofs[s & 3], 128 * (s >> 2)), qreg[s], sacc);

      float x[16];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int n = 8 * (e >> 2) + 4 * g + (e & 3);
        x[e] = (tile_base + n < r1) ? sacc[e] * p.scale_log2 : -__builtin_inff();
        tmax = fmaxf(tmax, x[e]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));

      // -- lazy rescale: only when the tile max passes the used max by > threshold
      const bool need = tmax > m + kRescaleThreshold;
      if (__any(need)) {
        const float mnew = need ? tmax : m;
        const float alpha = need ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int vb = 0; vb < 16; ++vb) acc[vb] *= alpha;
      }
      const float mu = (m == -__builtin_inff()) ? 0.f : m;

      // -- P = 2^(x - m), rounded to the input type: B operand of P·V
      u32x4 pk[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = __builtin_amdgcn_exp2f(x[8 * kt + j] - mu);
          lsum += pv[j];
        }
        pk[kt].x = pack2<DT>(pv[0], pv[1]);
        pk[kt].y = pack2<DT>(pv[2], pv[3]);
        pk[kt].z = pack2<DT>(pv[4], pv[5]);
        pk[kt].w = pack2<DT>(pv[6], pv[7]);
      }

      // -- Oᵀ[v][h] += Vᵀ[v][n] Pᵀ[n][h]
#pragma unroll
      for (int vb = 0; vb < 16; ++vb) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          acc[vb] = mfma32<DT>(lds_get(buf + vofs[kt][vb & 1], 2048 * vb), pk[kt], acc[vb]);
        }
      }
    }

    if (more) store_tile(lds + ((t + 1) & 1) * kBufBytes, wave, lane, tr);
    __syncthreads();
  }

  if (!wave_active) return;

  // ---- epilogue: normalise; write final output or the split partial --------
  const float ltot = lsum + __shfl_xor(lsum, 32);
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

hipError_t launch_split(const SplitParams& p, int dtype, bool paged, int grid_x, int grid_y,
                        hipStream_t stream) {
  const dim3 grid(grid_x, grid_y), block(kThreads);
  if (dtype == MLA_DTYPE_F16) {
    if (paged) hipLaunchKernelGGL((split_kernel<MLA_DTYPE_F16, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((split_kernel<MLA_DTYPE_F16, false>), grid, block, 0, stream, p);
  } else {
    if (paged) hipLaunchKernelGGL((split_kernel<MLA_DTYPE_BF16, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((split_kernel<MLA_DTYPE_BF16, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int dtype, int batch, hipStream_t stream) {
  const dim3 grid((p.heads + 3) / 4, batch), block(256);
  if (dtype == MLA_DTYPE_F16) hipLaunchKernelGGL(combine_kernel<MLA_DTYPE_F16>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(combine_kernel<MLA_DTYPE_BF16>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
