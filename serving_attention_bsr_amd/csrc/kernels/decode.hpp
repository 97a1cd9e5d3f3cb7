// decode.hpp -- VALU attention body for work items with few folded query rows.
//
// Terms "GQA head-group fusion" of the FlashInfer explainer page (paper
// Appendix A, Figure 11): the g query heads that share a KV head are folded into
// the query dimension, so one load of a KV row serves the whole group.  Core
// mechanism 4 (paper section 3.2.2): with a query tile below the matrix-core
// minimum the body runs on the vector ALUs.  Background (paper section 2.1):
// decode is memory-bound, so the body is organised around the KV stream.
//
// Mapping on a 64-lane wavefront: a KV row of D elements is read by D/16 lanes,
// each holding 16 elements (two 16-byte loads for bf16, four for fp32), so a
// wavefront reads 1024/D rows per step.  Each lane keeps the folded query rows
// for its 16 elements in registers, so every KV byte is loaded once, into the
// lanes that use it, and serves all ROWS query rows: the page gather lands
// straight in registers; LDS is used only to combine the four wavefronts at the
// end of an item.  Each group of D/16 lanes runs its own online softmax over the
// rows it reads (running max and sum in base 2); groups and wavefronts are
// combined with ⊕ at the end of the item.
//
// Page gather (Core mechanism 1, paper section 3.1.1): key tau of the block row
// is slot tau % P of page kv_indices[page_begin + tau / P].  Page ids are loaded
// three steps ahead of the arithmetic and K/V rows two steps ahead, so a
// wavefront keeps two steps of KV loads in flight while it computes.  Keys past
// the chunk are clamped to its last key and masked, so no unused slot is ever
// read.
#pragma once

#include "common.hpp"

namespace bsr {

// KV8: K and V are OCP FP8 E4M3 codes (one byte per element) while Q and O are
// bf16; a lane then holds 16 consecutive elements of a KV row in one 16-byte load,
// and its 16 query elements are the same ones (two 16-byte loads of bf16).  The
// codes are converted exactly (E4M3 values are bf16 values) by the gfx950
// conversion instruction, whose decoding of all 256 codes was checked against the
// format on the GPU.
// VAR: the plan may carry ALiBi slopes and tree masks (instances without it keep
// the plain code, whose registers are tight).
template <int D, bool BF16, int ROWS, int TB, bool CAP, bool KV8 = false, bool VAR = false>
struct DecodeBody {
  static_assert(!KV8 || BF16, "an FP8 K/V cache has bf16 queries");
  static constexpr int LPT = D / 16;                 // lanes per KV row
  static constexpr int NG = 64 / LPT;                // KV rows per wavefront step slot
  static constexpr int QSZ = BF16 ? 2 : 4;           // Q / O element bytes
  static constexpr int ESZ = KV8 ? 1 : QSZ;          // K / V element bytes
  static constexpr int NLD = 16 * ESZ / 16;          // 16-byte K/V loads per row per lane
  static constexpr int EPL = 16 / ESZ;               // elements per 16-byte K/V load
  static constexpr int QLD = 16 * QSZ / 16;          // 16-byte Q loads per row per lane
  static constexpr int TILE = NG * TB;               // keys per wavefront step
  static constexpr int LDS_FLOATS = kWaves * ROWS * (D + 2);
  static_assert(D == 64 || D == 128 || D == 256, "head_dim");

  struct Pids {
    uint32_t row[TB];  // KV row index in the pool: (page * H_kv + head) * P + slot
  };
  struct Kv {
    uint4 k[TB][NLD];
    uint4 v[TB][NLD];
  };

  // element index of accumulator slot j of lane chunk c
  static __device__ __forceinline__ int elem(int c, int j) {
    return (j / EPL) * (LPT * EPL) + c * EPL + (j % EPL);
  }

  static __device__ __forceinline__ void load_pids(const RunParams& p, __amdgpu_buffer_rsrc_t ir,
                                                   const WorkItem& it, int tile, int grp, Pids& out) {
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      int tau = it.kv_begin + tile * TILE + i * NG + grp;
      tau = min(tau, it.kv_end - 1);
      const uint32_t pl = div_magic(static_cast<uint32_t>(tau), p.page_magic, p.page_shift);
      const uint32_t slot = static_cast<uint32_t>(tau) - pl * static_cast<uint32_t>(p.page_size);
      const uint32_t page = load_u32(ir, it.page_begin + static_cast<int32_t>(pl));
      // (page * H_kv + head) * P + slot
      out.row[i] = page * static_cast<uint32_t>(p.h_kv * p.page_size) +
                   (static_cast<uint32_t>(it.kv_head * p.page_size) + slot);
    }
  }

  // K/V rows through structured buffer resources over rows of D elements.
  static __device__ __forceinline__ void load_kv(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int c,
                                                 const Pids& ids, Kv& out) {
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      const int row = static_cast<int>(ids.row[i]);
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        out.k[i][j] = __builtin_bit_cast(uint4, bsr_struct_load_b128(kr, row, c * 16 + j * (LPT * 16), 0, 0));
        out.v[i][j] = __builtin_bit_cast(uint4, bsr_struct_load_b128(vr, row, c * 16 + j * (LPT * 16), 0, 0));
      }
    }
  }

  struct State {
    float acc[ROWS][16];
    float m[ROWS];
    float l[ROWS];
  };


  // The state of the lane LEVEL lanes away in the ⊕ across lane groups, as a pair
  // (a, b) to be combined.  Below 16, a rotation by LEVEL within each 16 lanes (the
  // partner keeps this lane's chunk index lane % LPT; rotations by LPT, 2 LPT, ...
  // reach all groups of the 16): a = own value, b = the partner's.  At 16 and 32
  // the lane-half swaps hand both partners the same pair, in lane order.  No LDS.
  template <int LEVEL>
  static __device__ __forceinline__ void partner(float x, float& a, float& b) {
    if constexpr (LEVEL >= 16) {
      lane_pair<LEVEL>(x, a, b);
    } else {
      a = x;
      b = dpp_mov<0x120 + LEVEL>(x);  // row_ror:LEVEL
    }
  }

  template <int LEVEL>
  static __device__ __forceinline__ void merge_groups(State& st) {
    if constexpr (LEVEL < 64) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float ma, mb, la, lb;
        partner<LEVEL>(st.m[r], ma, mb);
        partner<LEVEL>(st.l[r], la, lb);
        const float m_new = __builtin_fmaxf(ma, mb);
        const float m_use = m_new == kNegInf ? 0.0f : m_new;
        const float fa = fast_exp2(ma - m_use);
        const float fb = fast_exp2(mb - m_use);
        st.l[r] = la * fa + lb * fb;
        st.m[r] = m_new;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float xa, xb;
          partner<LEVEL>(st.acc[r][e], xa, xb);
          st.acc[r][e] = xa * fa + xb * fb;
        }
      }
      merge_groups<LEVEL * 2>(st);
    }
  }


  static __device__ __forceinline__ float dot_row(const uint4 (&q)[QLD], const uint4 (&k)[NLD]) {
    float s = 0.0f;
    if constexpr (KV8) {
      const uint32_t kw[4] = {k[0].x, k[0].y, k[0].z, k[0].w};
      const uint32_t qw[8] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        s = dot2_bf16(qw[2 * w], e4m3x2_to_bf16x2<false>(kw[w]), s);
        s = dot2_bf16(qw[2 * w + 1], e4m3x2_to_bf16x2<true>(kw[w]), s);
      }
      return s;
    }
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      if constexpr (BF16) {
        s = dot2_bf16(q[j].x, k[j].x, s);
        s = dot2_bf16(q[j].y, k[j].y, s);
        s = dot2_bf16(q[j].z, k[j].z, s);
        s = dot2_bf16(q[j].w, k[j].w, s);
      } else {
        s = __builtin_fmaf(__uint_as_float(q[j].x), __uint_as_float(k[j].x), s);
        s = __builtin_fmaf(__uint_as_float(q[j].y), __uint_as_float(k[j].y), s);
        s = __builtin_fmaf(__uint_as_float(q[j].z), __uint_as_float(k[j].z), s);
        s = __builtin_fmaf(__uint_as_float(q[j].w), __uint_as_float(k[j].w), s);
      }
    }
    return s;
  }

  static __device__ __forceinline__ void unpack_v(const uint4 (&v)[NLD], float (&out)[16]) {
    if constexpr (KV8) {
      const uint32_t vw[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(vw[w]), false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(vw[w]), true);
        out[4 * w] = lo[0];
        out[4 * w + 1] = lo[1];
        out[4 * w + 2] = hi[0];
        out[4 * w + 3] = hi[1];
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if constexpr (BF16) {
          out[j * 8 + 2 * t] = bf16_lo(w[t]);
          out[j * 8 + 2 * t + 1] = bf16_hi(w[t]);
        } else {
          out[j * 4 + t] = __uint_as_float(w[t]);
        }
      }
    }
  }

  // One tile of keys.  live = false masks every key: the update is then an exact
  // no-op (alpha = 1, p = 0 against finite values).
  static __device__ __forceinline__ void step(const RunParams& p, const WorkItem& it, int tile,
                                              int grp, bool live, const uint4 (&q)[ROWS][QLD],
                                              const Kv& kv, const Variant& var, State& st) {
    float s[TB][ROWS];
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
      for (int r = 0; r < ROWS; ++r) s[i][r] = group_sum<LPT>(dot_row(q[r], kv.k[i]));
    const int g = p.group;
    const int step_base = it.kv_begin + tile * TILE;
    // ALiBi: key tau of row r (head kv_head g + r % g, token r / g) gains
    // slope (tau - pos), before the soft-cap; the slopes are read here (uniform
    // loads) rather than held for the whole item
    if (VAR && var.has_alibi) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const float slope = load_invariant(var.alibi + it.kv_head * g + r % g);
        const int pos = it.q_pos + r / g;
#pragma unroll
        for (int i = 0; i < TB; ++i)
          s[i][r] = __builtin_fmaf(slope, static_cast<float>(step_base + i * NG + grp - pos), s[i][r]);
      }
    }
    // logits in base 2 are c * s: without a soft-cap the scale is folded into the
    // exponent's fma (c > 0, so the maximum of the raw scores gives the maximum);
    // with one, s is first mapped to cap * tanh(s / cap) in base 2
    const float c = CAP ? 1.0f : p.scale_log2;
    if constexpr (CAP) {
#pragma unroll
      for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int r = 0; r < ROWS; ++r) s[i][r] = p.cap_log2 * tanh_exp(s[i][r] * p.sm_scale * p.cap_inv);
    }
    // masks only on steps that reach past the chunk end or the causal limit of the
    // first row, below the sliding-window start of the last token, or into the
    // tree-masked new tokens (a real branch: most steps lie inside)
    if (!live || step_base + TILE > it.kv_end || step_base + TILE - 1 > it.causal_limit ||
        step_base < it.window_lo + it.qo_count || (VAR && step_base + TILE > it.tree_lo)) {
      asm volatile("");
      const bool tree = VAR && it.tree_lo != kNoTree;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        // the tree-mask row of this row's token (read on masked steps only)
        const uint64_t trow = tree ? load_invariant(var.tree + it.qo_begin + r / g) : ~uint64_t(0);
#pragma unroll
        for (int i = 0; i < TB; ++i) {
          const int tau = step_base + i * NG + grp;
          const bool in_chunk = live && tau < it.kv_end;
          const bool in_tree = tau < it.tree_lo || ((trow >> ((tau - it.tree_lo) & 63)) & 1) != 0;
          const bool visible =
              in_chunk && tau <= it.causal_limit + r / g && tau >= it.window_lo + r / g && in_tree;
          s[i][r] = visible ? s[i][r] : kNegInf;
        }
      }
    }
    // lazy reference maximum (see lazy_max): the accumulators are rescaled, in a
    // real branch, only on steps where some row's reference moved
    float alpha[ROWS];
    bool moved = false;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      float mx = s[0][r];
#pragma unroll
      for (int i = 1; i < TB; ++i) mx = __builtin_fmaxf(mx, s[i][r]);
      const float m_new = lazy_max(st.m[r], mx * c);
      const float m_use = m_new == kNegInf ? 0.0f : m_new;
      alpha[r] = m_new == st.m[r] ? 1.0f : fast_exp2(st.m[r] - m_use);
      moved |= m_new != st.m[r];
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        s[i][r] = fast_exp2(__builtin_fmaf(s[i][r], c, -m_use));
        psum += s[i][r];
      }
      st.l[r] = st.l[r] * alpha[r] + psum;
      st.m[r] = m_new;
    }
    if (__ballot(moved) != 0) {
      asm volatile("");
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int e = 0; e < 16; ++e) st.acc[r][e] *= alpha[r];
    }
    if constexpr (KV8) {
      // two keys at a time: acc += p_i v_i + p_j v_j as one bf16 dot product per
      // element; the codes of the two keys are interleaved byte by byte and
      // converted to (v_i, v_j) bf16 pairs, the probabilities rounded to bf16
      // pairs (the running sum keeps them unrounded)
      static_assert(TB % 2 == 0, "keys in pairs");
#pragma unroll
      for (int i = 0; i < TB; i += 2) {
        uint32_t pp[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) pp[r] = pack_bf16x2(s[i][r], s[i + 1][r]);
        const uint32_t va[4] = {kv.v[i][0].x, kv.v[i][0].y, kv.v[i][0].z, kv.v[i][0].w};
        const uint32_t vb[4] = {kv.v[i + 1][0].x, kv.v[i + 1][0].y, kv.v[i + 1][0].z, kv.v[i + 1][0].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // bytes (a0, b0, a1, b1) and (a2, b2, a3, b3) of elements 4w .. 4w + 3
          const uint32_t lo = __builtin_amdgcn_perm(vb[w], va[w], 0x05010400u);
          const uint32_t hi = __builtin_amdgcn_perm(vb[w], va[w], 0x07030602u);
          const uint32_t pair[4] = {e4m3x2_to_bf16x2<false>(lo), e4m3x2_to_bf16x2<true>(lo),
                                    e4m3x2_to_bf16x2<false>(hi), e4m3x2_to_bf16x2<true>(hi)};
#pragma unroll
          for (int r = 0; r < ROWS; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) st.acc[r][4 * w + j] = dot2_bf16(pair[j], pp[r], st.acc[r][4 * w + j]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        float v[16];
        unpack_v(kv.v[i], v);
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
          for (int e = 0; e < 16; ++e) st.acc[r][e] = __builtin_fmaf(s[i][r], v[e], st.acc[r][e]);
      }
    }
  }

  // Attention of one work item; result in the workgroup-combined (O, log2-sum-exp)
  // handed to `emit(row, d_pair, o0, o1, lse2)`.
  template <typename Emit>
  static __device__ void run(const RunParams& p, const WorkItem& it, const Variant& var, float* lds, Emit&& emit) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps loops scalar
    const int c = lane % LPT;
    const int grp = lane / LPT;
    const int g = p.group;
    const int rows_valid = it.qo_count * g;

    // folded query rows: row r = token (r / g) of the tile, head kv_head * g + r % g
    uint4 q[ROWS][QLD];
    {
      const uint8_t* qb = static_cast<const uint8_t*>(p.q);
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        if (r < rows_valid) {
          const int64_t qrow = static_cast<int64_t>(it.qo_begin + r / g) * p.h_qo +
                               it.kv_head * g + r % g;
          if constexpr (KV8) {
            // this lane's 16 consecutive elements c * 16 .. c * 16 + 15
            const uint8_t* src = qb + qrow * (D * QSZ) + c * 32;
            q[r][0] = *reinterpret_cast<const uint4*>(src);
            q[r][1] = *reinterpret_cast<const uint4*>(src + 16);
          } else {
            const uint8_t* src = qb + qrow * (D * QSZ) + c * 16;
#pragma unroll
            for (int j = 0; j < QLD; ++j) q[r][j] = *reinterpret_cast<const uint4*>(src + j * (LPT * 16));
          }
        } else {
#pragma unroll
          for (int j = 0; j < QLD; ++j) q[r][j] = make_uint4(0, 0, 0, 0);
        }
      }
    }

    State st;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      st.m[r] = kNegInf;
      st.l[r] = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) st.acc[r][e] = 0.0f;
    }

    // Tiles wave, wave + 4, ... of the item; local tile j of this wavefront.
    // Pipeline (issue order is what the in-order load counter sees): step j
    // issues the page ids of tile j+3, then K/V of tile j+2 (its ids arrived a
    // step ago, and were issued before K/V of tile j+1, so waiting for them
    // leaves tile j+1 in flight), then computes tile j.  The loop starts at
    // j = -3 with every key masked while j < 0, so every load is issued and
    // consumed by the one loop body on every path (a separate prologue, or a
    // branch around the arithmetic, would leave loads pending into registers
    // the loop head reuses and force a full wait there).  The id buffers start
    // at the row of the chunk's first key, and loads past the end are clamped to
    // its last key, so every load is in bounds and no load sits behind a branch.
    const __amdgpu_buffer_rsrc_t krs = row_rsrc(p.k_pool, D * ESZ);
    const __amdgpu_buffer_rsrc_t vrs = row_rsrc(p.v_pool, D * ESZ);
    const __amdgpu_buffer_rsrc_t irs = row_rsrc(p.kv_indices, 0);
    const int ntok = it.kv_end - it.kv_begin;
    const int ntiles = (ntok + TILE - 1) / TILE;
    const int nt_w = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
    if (nt_w > 0) {
      Pids p0, p1, p2;
      Kv k0 = {}, k1 = {}, k2 = {};  // warm-up steps read these before any load lands
      {
        const uint32_t first = load_u32(irs, it.page_begin + it.kv_begin / p.page_size);
        const uint32_t row0 = (first * static_cast<uint32_t>(p.h_kv) + static_cast<uint32_t>(it.kv_head)) *
                                  static_cast<uint32_t>(p.page_size) +
                              static_cast<uint32_t>(it.kv_begin % p.page_size);
#pragma unroll
        for (int i = 0; i < TB; ++i) p2.row[i] = row0;
      }
      const int t0 = wave;
      int j = -3;
      asm volatile("" : "+s"(j));  // keep the warm-up steps inside the loop
      while (true) {
        load_pids(p, irs, it, t0 + (j + 3) * kWaves, grp, p0);
        load_kv(krs, vrs, c, p2, k2);
        step(p, it, t0 + j * kWaves, grp, j >= 0, q, k0, var, st);
        if (++j >= nt_w) break;
        load_pids(p, irs, it, t0 + (j + 3) * kWaves, grp, p1);
        load_kv(krs, vrs, c, p0, k0);
        step(p, it, t0 + j * kWaves, grp, j >= 0, q, k1, var, st);
        if (++j >= nt_w) break;
        load_pids(p, irs, it, t0 + (j + 3) * kWaves, grp, p2);
        load_kv(krs, vrs, c, p1, k1);
        step(p, it, t0 + j * kWaves, grp, j >= 0, q, k2, var, st);
        if (++j >= nt_w) break;
      }
    }

    // ⊕ across the lane groups of this wavefront (lanes with the same lane % LPT)
    merge_groups<LPT>(st);

    // ⊕ across the four wavefronts through LDS: [wave][row][D] accumulators then
    // [wave][row] (m, l)
    float* lacc = lds;
    float* lml = lds + kWaves * ROWS * D;
    if (grp == 0) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int e = 0; e < 16; ++e) lacc[(wave * ROWS + r) * D + elem(c, e)] = st.acc[r][e];
      if (c == 0) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          lml[(wave * ROWS + r) * 2] = st.m[r];
          lml[(wave * ROWS + r) * 2 + 1] = st.l[r];
        }
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < ROWS * (D / 2); idx += kWgThreads) {
      const int r = idx / (D / 2);
      const int d = (idx % (D / 2)) * 2;
      if (r >= rows_valid) continue;
      float mw[kWaves];
      float big = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mw[w] = lml[(w * ROWS + r) * 2];
        big = __builtin_fmaxf(big, mw[w]);
      }
      const float m_use = big == kNegInf ? 0.0f : big;
      float lsum = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float a = fast_exp2(mw[w] - m_use);
        lsum += lml[(w * ROWS + r) * 2 + 1] * a;
        o0 += lacc[(w * ROWS + r) * D + d] * a;
        o1 += lacc[(w * ROWS + r) * D + d + 1] * a;
      }
      if (lsum > 0.0f) {
        const float inv = 1.0f / lsum;
        emit(r, d, o0 * inv, o1 * inv, big + fast_log2(lsum));
      } else {
        emit(r, d, 0.0f, 0.0f, kNegInf);
      }
    }
    __syncthreads();
  }
};

}  // namespace bsr
