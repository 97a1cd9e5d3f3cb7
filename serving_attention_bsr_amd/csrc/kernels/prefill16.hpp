// prefill16.hpp -- MFMA attention body with 16 folded rows per wavefront, for
// head_dim 256, and for the 64-row tiles of short query rows at head_dim 128.
//
// Same method as prefill.hpp (Core mechanisms 3 and 4 of the FlashInfer explainer
// page, paper sections 3.2 and 3.2.2; GQA folding, paper Appendix A): gathered KV
// tiles in LDS, S^T = K Q^T and O^T += V^T P^T on the matrix cores, base-2 online
// softmax in between.  At D = 256 a 32-row wavefront needs a 128-float
// accumulator and 64 registers of Q per lane, which leaves one wavefront per
// SIMD.  Here each wavefront owns 16 rows and uses v_mfma_f32_16x16x32_bf16, so
// the accumulator is 64 floats and Q 32 registers: two workgroups fit per CU and
// one workgroup's softmax and gather overlap the other's products.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (measured on gfx950 with a probe):
// A: lane l holds A[l % 16][8 (l / 16) + j], B: lane l holds B[8 (l / 16) + j][l % 16]
// (j = 0..7), C: lane l holds C[4 (l / 16) + i][l % 16] (i = 0..3).
//
// A workgroup (4 wavefronts) owns 64 folded rows; wavefront w owns rows
// 16w..16w+15.  Per tile of 32 keys:
//   * K and V rows are gathered by buffer loads that write LDS directly (one tile
//     ahead, page ids two tiles ahead) into one of two row-major LDS buffers whose
//     16-byte chunks are permuted per row against bank conflicts;
//   * S^T = K Q^T per 16-key block kb: each lane then holds keys
//     16 kb + 4 (l / 16) + i of query row l % 16, so a row's values sit in the four
//     lanes l % 16 + 16 q and the row max and sum take two cross-lane steps;
//   * O^T += V^T P^T with one 32-key MFMA step per 16-row block of D: the P
//     registers are the B operand as the S^T results left them (MFMA k index
//     8 (l / 16) + j is key 4 (l / 16) + j for j < 4 and 16 + 4 (l / 16) + j - 4
//     otherwise), and V^T is read in that key order with the LDS transpose read.
#pragma once

#include "common.hpp"

// k-steps per group of the S^T pipeline
#ifndef BSR_QK16_J
#define BSR_QK16_J 2
#endif

namespace bsr {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// PAGE1: every page holds one key, so a key's page is its own position.
// VAR: the plan may carry ALiBi slopes and tree masks.
template <int D, bool CAP, bool PAGE1 = false, bool VAR = false>
struct MfmaBody16 {
  static constexpr int BR = 64;            // folded rows per item
  static constexpr int BC = 32;            // keys per tile
  static constexpr int KB = BC / 16;       // 16-key blocks of S^T
  static constexpr int DK = D / 32;        // MFMA k-steps over D for S^T
  static constexpr int DB = D / 16;        // 16-row blocks of O^T
  static constexpr int NCH = D / 8;        // 16-byte chunks per row
  static constexpr int RPI = 64 / NCH;     // rows per 1 KB gather instruction
  static constexpr int NI = BC / RPI / kWaves;  // gather instructions per wavefront, tile and matrix
  // Unpadded tiles (row r at r * D elements, K then V) with the 16-byte chunks of
  // each row permuted: chunk c of row r sits in slot c ^ swz(r).  K is read one row
  // per lane, 16 lanes per pass at one chunk: swz_k puts 16 consecutive rows on
  // the 16 slots of 256 bytes.  V is read with the transpose read, 8 consecutive
  // keys x 32 bytes per half-wave: swz_v puts the 8 rows' 32-byte pairs of chunks
  // on 8 distinct eighths of the banks.
  static constexpr int STAGE = 2 * BC * D;  // bf16 elements of one buffer
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static constexpr int LDS_FLOATS = (LDS_BYTES + 3) / 4;
  static_assert(D == 256 || D == 128, "the 16-row body serves head_dim 256, and short tiles at 128");
  static_assert(NI * RPI * kWaves == BC, "whole gather instructions per wavefront");

  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

  static __device__ __forceinline__ int swz_k(int r) { return r % 16; }
  static __device__ __forceinline__ int swz_v(int r) { return 2 * (r % 8); }

  // Page ids loaded a tile ahead of their rows, kept as loaded (see MfmaBody::Rows)
  struct Rows {
    uint32_t page[NI];
    uint32_t off[NI];   // head * P + slot: row = page * (H_kv * P) + off
  };

  static __device__ __forceinline__ int lane_row(int wave, int lane, int n) {
    return RPI * (NI * wave + n) + lane / NCH;
  }

  static __device__ __forceinline__ void load_rows(const RunParams& p, __amdgpu_buffer_rsrc_t ir,
                                                   const WorkItem& it, int tile, int wave, int lane, Rows& out) {
    const int tau0 = it.kv_begin + tile * BC;
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int tau = min(tau0 + lane_row(wave, lane, n), it.kv_end - 1);
      if constexpr (PAGE1) {
        out.page[n] = load_u32(ir, it.page_begin + tau);
        out.off[n] = static_cast<uint32_t>(it.kv_head);
      } else {
        const uint32_t pl = div_magic(static_cast<uint32_t>(tau), p.page_magic, p.page_shift);
        const uint32_t slot = static_cast<uint32_t>(tau) - pl * static_cast<uint32_t>(p.page_size);
        out.page[n] = load_u32(ir, it.page_begin + static_cast<int32_t>(pl));
        out.off[n] = static_cast<uint32_t>(it.kv_head * p.page_size) + slot;
      }
    }
  }

  // Gather this lane's rows N0 <= n < N1 of a tile's K and V into a buffer (K at
  // buf, V at buf + BC * D).
  template <int N0 = 0, int N1 = NI>
  static __device__ __forceinline__ void gather(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                                uint32_t rows_per_page, const Rows& rows, uint16_t* buf, int wave,
                                                int lane) {
    const int slot = lane % NCH;
#pragma unroll
    for (int n = N0; n < N1; ++n) {
      const int r = lane_row(wave, lane, n);
      const int row = static_cast<int>(rows.page[n] * rows_per_page + rows.off[n]);
      uint16_t* dst = buf + (NI * wave + n) * 512;
      lds_gather_b128(kr, dst, row, 16 * (slot ^ swz_k(r)));
      lds_gather_b128(vr, dst + BC * D, row, 16 * (slot ^ swz_v(r)));
    }
  }

  static __device__ __forceinline__ i16x4_t read_tr(const uint16_t* addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(const_cast<uint16_t*>(addr)));
  }

  // S^T = K Q^T: block kb covers keys 16 kb .. 16 kb + 15.  A two-stage pipeline
  // over groups of QK_J k-steps, as in MfmaBody::qk: the K operands of group g + 1
  // are read from LDS, then the products of group g issue with the block chains
  // alternating; scheduling barriers keep that order (left to itself the scheduler
  // sinks each read next to its product, one LDS round trip per product).
  static constexpr int QK_J = BSR_QK16_J;
  static_assert(DK % QK_J == 0, "whole groups of k-steps");
  static __device__ __forceinline__ void qk(const uint16_t* lk, const bf16x8_t (&qreg)[DK], int r16, int grp,
                                            f32x4_t (&s)[KB]) {
    constexpr int G = DK / QK_J;
    auto read = [&](int ks, int kb) -> bf16x8_t {
      // row 16 kb + r16, chunk 4 ks + grp (swz_k(16 kb + r16) == swz_k(r16))
      return __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const u32x4_t*>(lk + (16 * kb + r16) * D + 8 * ((4 * ks + grp) ^ swz_k(r16))));
    };
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8_t a[2][QK_J][KB];  // [stage][k-step of the group][block]
#pragma unroll
    for (int j = 0; j < QK_J; ++j)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) a[0][j][kb] = read(j, kb);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int cur = g & 1;
      if (g + 1 < G) {
#pragma unroll
        for (int j = 0; j < QK_J; ++j)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) a[cur ^ 1][j][kb] = read(QK_J * (g + 1) + j, kb);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < QK_J; ++j)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[cur][j][kb], qreg[QK_J * g + j], s[kb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ALiBi bias, soft-cap (base 2) and the chunk-end / causal / window / tree mask
  // of tile t (see MfmaBody::cap_and_mask).
  static __device__ __forceinline__ void cap_and_mask(const RunParams& p, const WorkItem& it, int t, int t_local,
                                                      int grp, bool alibi, float slope, int pos, uint64_t tm,
                                                      f32x4_t (&s)[KB]) {
    const int tile_base = it.kv_begin + t * BC;
    if (VAR && alibi) {
      // key 16 kb + 4 grp + i of the tile gains slope (key - pos)
      const float base = static_cast<float>(tile_base + 4 * grp - pos);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kb][i] = __builtin_fmaf(slope, base + static_cast<float>(16 * kb + i), s[kb][i]);
    }
    if constexpr (CAP) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kb][i] = p.cap_log2 * tanh_exp(s[kb][i] * p.sm_scale * p.cap_inv);
    }
    if (tile_base + BC > it.kv_end || tile_base + BC - 1 > it.causal_limit || tile_base < it.window_lo + it.qo_count ||
        (VAR && tile_base + BC > it.tree_lo)) {
      asm volatile("");  // keep this a branch: only boundary tiles pay for the mask
      // key 16 kb + 4 grp + i of the tile is visible up to the chunk end and this
      // row's causal limit
      const int lim = min(it.kv_end - 1, it.causal_limit + t_local) - tile_base - 4 * grp;
      // and from this row's sliding-window start on
      const int low = max(it.window_lo + t_local, it.kv_begin) - tile_base - 4 * grp;
      // and, among the tree-masked new tokens, where the token's tree row allows
      const int tlo = VAR ? it.tree_lo - tile_base - 4 * grp : kNoTree;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kr = 16 * kb + i;
          const bool tree_hides = kr >= tlo && ((tm >> ((kr - tlo) & 63)) & 1) == 0;
          if (kr > lim || kr < low || tree_hides) s[kb][i] = kNegInf;
        }
    }
  }

  // Online softmax of one tile; returns the accumulator factor (exactly 1 when
  // the reference stays).  m_run is the row's reference maximum (lazy, see
  // lazy_max; the same in the row's four lanes), l_run this lane's share of the
  // running sum.
  static __device__ __forceinline__ float softmax(const f32x4_t (&s)[KB], float c, float& m_run, float& l_run,
                                                  bf16x8_t& pb) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = __builtin_fmaxf(mx, s[kb][i]);
    mx = pair_max<32>(pair_max<16>(mx)) * c;
    const float m_new = lazy_max(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = m_new == m_run ? 1.0f : fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(__builtin_fmaf(s[kb][i], c, -m_use));
        psum += e;
        pb[4 * kb + i] = static_cast<__bf16>(e);
      }
    }
    l_run = l_run * alpha + psum;
    return alpha;
  }

  static __device__ __forceinline__ void rescale(float alpha, f32x4_t (&acc)[DB]) {
    if (__ballot(alpha != 1.0f) != 0) {
      asm volatile("");  // a real branch: most tiles leave the running maxima unchanged
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[db][i] *= alpha;
    }
  }

  // O^T += V^T P^T.  The A operand lane (16 db + l % 16, group l / 16) needs V^T at
  // keys 4 (l / 16) + 0..3, then 16 + 4 (l / 16) + 0..3.  With the transpose read,
  // lane l of a 16-lane group receives element l & 3 of the 4-element rows
  // addressed by lanes 4 e + l / 4, so lane s addresses key base + s / 4 at
  // d = 16 db + 4 (s & 3): key_off and d_off below.
  static __device__ __forceinline__ void pv(const uint16_t* lv, const bf16x8_t& pb, int key_off, int d_off,
                                            f32x4_t (&acc)[DB]) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      // chunk (16 db + d_off) / 8 of rows key_off and 16 + key_off (same swizzle)
      const int at = 8 * ((2 * db + d_off / 8) ^ swz_v(key_off)) + d_off % 8;
      const i16x4_t lo = read_tr(lv + key_off * D + at);
      const i16x4_t hi = read_tr(lv + (16 + key_off) * D + at);
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[db], 0, 0, 0);
    }
  }

  template <typename Emit>
  static __device__ void run(const RunParams& p, const WorkItem& it, const Variant& var, float* lds_f,
                             Emit&& emit) {
    uint16_t* lds_h = reinterpret_cast<uint16_t*>(lds_f);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15;     // query row of this lane within the wavefront
    const int grp = lane >> 4;     // lane group: k block of the operands, key quad of S^T
    const int g = p.group;
    const int rows_valid = it.qo_count * g;
    const int rho = wave * 16 + r16;
    const bool row_ok = rho < rows_valid;
    const int t_local = rho / g;
    const int key_off = 4 * grp + (r16 >> 2);
    const int d_off = 4 * (r16 & 3);
    // variant state of this lane's row: ALiBi slope and position, tree-mask row
    const bool alibi = VAR && var.has_alibi;
    const float slope = alibi && row_ok ? var.alibi[it.kv_head * g + rho % g] : 0.0f;
    const int pos = it.q_pos + t_local;
    const uint64_t tm =
        VAR && it.tree_lo != kNoTree && row_ok ? var.tree[it.qo_begin + t_local] : ~uint64_t(0);

    // Q rows as the B operand: Q[rho][32 ks + 8 grp + 0..7]
    bf16x8_t qreg[DK];
    {
      const uint16_t* qb = static_cast<const uint16_t*>(p.q);
      const int64_t qrow = static_cast<int64_t>(it.qo_begin + t_local) * p.h_qo + it.kv_head * g + rho % g;
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (row_ok) v = *reinterpret_cast<const u32x4_t*>(qb + qrow * D + 32 * ks + 8 * grp);
        qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
      }
    }

    f32x4_t acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = kNegInf;
    const float c = CAP ? 1.0f : p.scale_log2;
    float l_run = 0.0f;

    const __amdgpu_buffer_rsrc_t krs = row_rsrc(p.k_pool, D * 2);
    const __amdgpu_buffer_rsrc_t vrs = row_rsrc(p.v_pool, D * 2);
    const __amdgpu_buffer_rsrc_t irs = row_rsrc(p.kv_indices, 0);
    const int ntok = it.kv_end - it.kv_begin;
    const int ntiles = (ntok + BC - 1) / BC;
    const uint32_t rpp = static_cast<uint32_t>(p.h_kv * p.page_size);
    Rows rows;
    // Two buffers: tile t lives in buffer t % 2.  The gather of tile t + 1 and the
    // page ids of tile t + 2 are issued while tile t is computed and waited for at
    // the next step.
    if (ntiles > 0) {
      load_rows(p, irs, it, 0, wave, lane, rows);
      gather(krs, vrs, rpp, rows, lds_h, wave, lane);
      if (ntiles > 1) load_rows(p, irs, it, 1, wave, lane, rows);
    }
    // One tile step: lk is the buffer holding tile t, nb the other one.
    auto tile = [&](int t, const uint16_t* lk, uint16_t* nb) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      if (t + 1 < ntiles) gather<0, NI / 2>(krs, vrs, rpp, rows, nb, wave, lane);
      f32x4_t s[KB];
      qk(lk, qreg, r16, grp, s);
      if (t + 1 < ntiles) {
        gather<NI / 2, NI>(krs, vrs, rpp, rows, nb, wave, lane);
        if (t + 2 < ntiles) load_rows(p, irs, it, t + 2, wave, lane, rows);
      }
      cap_and_mask(p, it, t, t_local, grp, alibi, slope, pos, tm, s);
      bf16x8_t pb;
      const float alpha = softmax(s, c, m_run, l_run, pb);
      rescale(alpha, acc);
      pv(lk + BC * D, pb, key_off, d_off, acc);
    };
    // tiles in pairs: fixed buffer offsets for each step's LDS reads
    for (int t = 0; t < ntiles; t += 2) {
      tile(t, lds_h, lds_h + STAGE);
      if (t + 1 < ntiles) tile(t + 1, lds_h + STAGE, lds_h);
    }

    // result: this lane holds O^T[16 db + 4 grp + i][rho]; the row's sum is spread
    // over its four lanes
    const float l_tot = pair_sum<32>(pair_sum<16>(l_run));
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse2 = l_tot > 0.0f ? m_run + fast_log2(l_tot) : kNegInf;
    if (row_ok) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 16 * db + 4 * grp;
        emit(rho, d, acc[db][0] * inv, acc[db][1] * inv, lse2);
        emit(rho, d + 2, acc[db][2] * inv, acc[db][3] * inv, lse2);
      }
    }
    __syncthreads();  // LDS free for the next item
  }
};

}  // namespace bsr
