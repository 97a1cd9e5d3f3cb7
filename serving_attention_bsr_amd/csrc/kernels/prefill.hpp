// prefill.hpp -- MFMA attention body for work items with many folded query rows.
//
// Core mechanism 3 of the FlashInfer explainer page (paper section 3.2): scattered
// KV tiles are gathered into contiguous on-chip tiles, after which sparse and
// dense share one dense body.  Core mechanism 4 (paper section 3.2.2): tiles of at
// least 16 query rows use the matrix cores.  Terms "GQA head-group fusion" (paper
// Appendix A): the g query heads of a KV head are folded into the query rows, so a
// tile of 128 folded rows is 128/g tokens and one KV tile serves all of them.
// Reproduction section (paper section 4.2): prefill runs with a causal mask.
//
// gfx950 mapping.  A workgroup (4 wavefronts) owns 128 folded rows; wavefront w
// owns rows 32w..32w+31.  Per tile of 64 keys:
//   * the workgroup gathers the keys' K and V rows page by page with 16-byte
//     buffer loads that write LDS directly (one tile ahead; page ids two tiles
//     ahead), row-major into one of two LDS buffers, so that one barrier per tile
//     suffices and no register or LDS-store instruction carries the tile; the
//     16-byte chunks of each row are permuted so that the reads below hit
//     distinct banks;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the
//     wavefront's Q rows, held in registers for the whole item): each lane then
//     holds one query column and 16 keys of each 32-key block, so the softmax max
//     and sums are in-lane (plus one exchange between the two lane halves);
//   * base-2 online softmax, soft-cap and the causal mask (only on tiles that
//     cross the diagonal or the chunk end);
//   * O^T += V^T P^T: the probabilities, converted to bf16, are the B operand in
//     exactly the registers the S^T result left them in; the A operand V^T is read
//     from the row-major V tile with the LDS transpose read (ds_read_b64_tr_b16),
//     whose lane addresses follow the key order of the P registers.
// The result leaves through the same emit callback as the decode body.
#pragma once

#include "common.hpp"

namespace bsr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// PAGE1: every page holds one key (page size 1, the radix-tree layout), so a key's
// page is its own position and no division is needed.
// VAR: the plan may carry ALiBi slopes and tree masks.
// KV8: K and V are OCP FP8 E4M3 codes (Q and O bf16; Appendix F of the paper, as
// the explainer page's Core mechanism 8 restates it: an FP8 cache with 16-bit
// queries, codes converted on chip).  Tiles then hold one byte per element (half
// the gather), and each operand read converts its 8 codes to bf16 exactly before
// the bf16 products: K rows with 8-byte reads, V^T with the gfx950 8-bit
// transpose read.
template <int D, bool CAP, bool PAGE1 = false, bool VAR = false, bool KV8 = false>
struct MfmaBody {
  static constexpr int BR = 128;           // folded rows per item
  static constexpr int BC = 64;            // keys per tile
  static constexpr int KB = BC / 32;       // 32-key blocks per tile
  static constexpr int DK = D / 16;        // MFMA k-steps over D for S^T
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
  static constexpr int RB = KV8 ? D : 2 * D;  // bytes of one K/V row
  static constexpr int NCH = RB / 16;      // 16-byte chunks per row
  static constexpr int RPI = 64 / NCH;     // rows per 1 KB gather instruction
  static constexpr int NI = BC / RPI / kWaves;  // gather instructions per wavefront, tile and matrix
  // Tiles are unpadded (row r at r * RB bytes, K then V) with the 16-byte chunks
  // of each row permuted: chunk c of row r sits in slot c ^ swz(r), which keeps every
  // gather instruction a contiguous 1 KB of LDS.  bf16: K is read one row per
  // lane, 16 lanes per pass, all at one chunk: swz_k puts 16 consecutive rows on the
  // 16 slots of 256 bytes (all 64 banks).  V is read with the transpose read, 4
  // consecutive keys x 64 bytes per half-wave: swz_v puts the 4 rows' 64-byte groups
  // on 4 distinct quarters of the banks.  FP8: see swz8.
  static constexpr int STAGE = 2 * BC * RB / 2;  // one buffer (K then V tile), in 16-bit units
  static constexpr int VOFF = BC * RB / 2;       // V tile inside a buffer, in 16-bit units
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static constexpr int LDS_FLOATS = (LDS_BYTES + 3) / 4;
  static_assert(D == 64 || D == 128, "head_dim (D = 256 uses the 16-row body)");
  static_assert(NI * RPI * kWaves == BC, "whole gather instructions per wavefront");

  // FP8 tiles (rows of D bytes): the K read of a half-wave takes 8 bytes at one
  // chunk of 32 consecutive rows, the V transpose read of a half-wave takes 2 x 8
  // bytes of two adjacent chunks from rows r0 + {0, 1, 2, 3, 8, 9, 10, 11}.  The
  // permutation below spreads the V read over all 64 banks and the K read over 16
  // slots (two rows per slot, the fewest 16-byte granularity allows): at D = 128
  // rows of one parity (same 128-byte half of 256 bytes) get slot bits (r2, r1, r3),
  // at D = 64 rows of one residue mod 4 get (r3, r2).
  static __device__ __forceinline__ int swz8(int r) {
    if constexpr (D == 128)
      return ((r >> 2) & 1) | (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2);
    else
      return ((r >> 2) & 1) | (((r >> 3) & 1) << 1);
  }
  static __device__ __forceinline__ int swz_k(int r) {
    if constexpr (KV8) return swz8(r);
    return (r / (16 / NCH)) % NCH;
  }
  static __device__ __forceinline__ int swz_v(int r) {
    if constexpr (KV8) return swz8(r);
    return 4 * ((r / (16 / NCH)) % (NCH / 4));
  }

  // Eight FP8 codes (in order) as the bf16x8 operand of one product.
  static __device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint2 w) {
    const u32x4_t v = {e4m3x2_to_bf16x2<false>(w.x), e4m3x2_to_bf16x2<true>(w.x), e4m3x2_to_bf16x2<false>(w.y),
                       e4m3x2_to_bf16x2<true>(w.y)};
    return __builtin_bit_cast(bf16x8_t, v);
  }

  // Page ids of this lane's rows, loaded a tile ahead of the rows themselves.  The
  // id is kept as loaded and the row index formed only when the rows are gathered:
  // arithmetic on the id right after its load would wait for every load issued
  // before it (the vector memory counter completes in order).
  struct Rows {
    uint32_t page[NI];
    uint32_t off[NI];   // head * P + slot: row = page * (H_kv * P) + off
  };

  // Row n of this lane in the tile: RPI rows per instruction, NI instructions per
  // wavefront, lane / NCH within the instruction.
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

  // Gather this lane's rows N0 <= n < N1 of a tile's K and V into the buffer at LDS
  // byte address buf (K at buf, V at buf + BC RB).  rows_per_page = H_kv * P: pool
  // rows between consecutive pages.
  static __device__ __forceinline__ void gather(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                                uint32_t rows_per_page, const Rows& rows, uint32_t buf, int wave,
                                                int lane, int n0 = 0, int n1 = NI) {
    const int slot = lane % NCH;
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      if (n < n0 || n >= n1) continue;  // n0, n1 are constants where this is inlined
      const int r = lane_row(wave, lane, n);
      const int row = static_cast<int>(rows.page[n] * rows_per_page + rows.off[n]);
      const uint32_t dst = buf + static_cast<uint32_t>(NI * wave + n) * 1024u;
      lds_gather_b128(kr, dst, row, 16 * (slot ^ swz_k(r)));
      lds_gather_b128(vr, dst + BC * RB, row, 16 * (slot ^ swz_v(r)));
    }
  }

  // Transpose read of 4 bf16 (one 8-byte half of a 16-byte chunk).
  static __device__ __forceinline__ i16x4_t read_tr(const uint16_t* addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(const_cast<uint16_t*>(addr)));
  }

  // 8-bit transpose read (FP8 V tiles).  Measured on gfx950 with an in-bounds
  // probe: within each 16-lane group, lane l receives as byte e (e = 0..7) byte
  // l & 7 of the 8 bytes addressed by lane 2 e + (l & 15) / 8 of its group.
  typedef int i32x2_t_ __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) i32x2_t_ lds_i32x2_t;
  static __device__ __forceinline__ uint2 read_tr8(const uint8_t* addr) {
    const i32x2_t_ v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(const_cast<uint8_t*>(addr)));
    return make_uint2(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]));
  }

  // ---- pieces of one tile step -------------------------------------------------

  // S^T = K Q^T for the tile whose K rows start at lk (32-key blocks kb).  bf16:
  // a two-stage pipeline over groups of two k-steps: the K operands of group g + 1
  // (both k-steps, every block) are read from LDS, then the products of group g
  // issue with the block chains alternating, so each product's operand was read a
  // whole group earlier and no product waits on the one just before it.  FP8: the
  // operands are converted after their reads, and the plain order (one block
  // after the other, each read next to its product) measured faster.
  // hook(h) runs DK / 2 times per tile (bf16: between the reads and the products
  // of group h): the next tile's gather is issued there a slice at a time, so that
  // its loads enter the address unit's queue between products, not in one burst.
  template <typename Hook>
  static __device__ __forceinline__ void qk(const uint16_t* lk, const bf16x8_t (&qreg)[DK], int col, int half,
                                            f32x16_t (&s)[KB], Hook&& hook) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
    if constexpr (KV8) {
      const uint8_t* lkb = reinterpret_cast<const uint8_t*>(lk);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
          // elements 16 ks + 8 half .. + 7 of row 32 kb + col: 8 bytes of chunk ks
          // (swz_k(32 kb + col) == swz_k(col): 32 rows apart)
          const bf16x8_t a = fp8x8_to_bf16x8(
              *reinterpret_cast<const uint2*>(lkb + (32 * kb + col) * RB + 16 * (ks ^ swz_k(col)) + 8 * half));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], s[kb], 0, 0, 0);
          if ((ks + 1) % (DK / 2) == 0 && kb * 2 + (ks + 1) / (DK / 2) - 1 < DK / 2)
            hook(2 * kb + (ks + 1) / (DK / 2) - 1);
        }
      }
      return;
    }
    constexpr int G = DK / 2;
    auto read = [&](int ks, int kb) -> bf16x8_t {
      const int r = 32 * kb + col;  // swz_k(r) == swz_k(col): 32 rows apart
      return __builtin_bit_cast(bf16x8_t,
                                *reinterpret_cast<const u32x4_t*>(lk + r * D + 8 * ((2 * ks + half) ^ swz_k(col))));
    };
    bf16x8_t a[2][2][KB];  // [stage][k-step of the group][block]
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) a[0][j][kb] = read(j, kb);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int cur = g & 1;
      if (g + 1 < G) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) a[cur ^ 1][j][kb] = read(2 * (g + 1) + j, kb);
      }
      hook(g);
      // The order above and below is kept as written: left to itself the machine
      // scheduler sinks every read next to its product and runs the block chains
      // one after the other, so each product waits out a whole LDS round trip.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][j][kb], qreg[2 * g + j], s[kb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ALiBi bias, soft-cap (base 2) and the chunk-end / causal / window / tree mask
  // of tile t.  slope and pos are this lane's row's ALiBi slope (unscaled-logit
  // units) and query position, tm its token's tree-mask row.
  static __device__ __forceinline__ void cap_and_mask(const RunParams& p, const WorkItem& it, int t, int t_local,
                                                      int half, bool alibi, float slope, int pos, uint64_t tm,
                                                      f32x16_t (&s)[KB]) {
    const int tile_base = it.kv_begin + t * BC;
    if (VAR && alibi) {
      // key 32 kb + 8 (r / 4) + 4 half + r % 4 of the tile gains slope (key - pos)
      const float base = static_cast<float>(tile_base + 4 * half - pos);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = __builtin_fmaf(slope, base + static_cast<float>(32 * kb + 8 * (r >> 2) + (r & 3)), s[kb][r]);
    }
    if constexpr (CAP) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = p.cap_log2 * tanh_exp(s[kb][r] * p.sm_scale * p.cap_inv);
    }
    if (tile_base + BC > it.kv_end || tile_base + BC - 1 > it.causal_limit || tile_base < it.window_lo + it.qo_count ||
        (VAR && tile_base + BC > it.tree_lo)) {
      // key 32 kb + 8 (r / 4) + 4 half + r % 4 of the tile is visible up to the
      // chunk end and this row's causal limit
      asm volatile("");  // keep this a branch: only boundary tiles pay for the mask
      const int lim = min(it.kv_end - 1, it.causal_limit + t_local) - tile_base - 4 * half;
      // and from this row's sliding-window start on
      const int low = max(it.window_lo + t_local, it.kv_begin) - tile_base - 4 * half;
      // and, among the tree-masked new tokens, where the token's tree row allows
      const int tlo = VAR ? it.tree_lo - tile_base - 4 * half : kNoTree;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = 32 * kb + 8 * (r >> 2) + (r & 3);
          const bool tree_hides = kr >= tlo && ((tm >> ((kr - tlo) & 63)) & 1) == 0;
          if (kr > lim || kr < low || tree_hides) s[kb][r] = kNegInf;
        }
    }
  }

  // Online softmax of one tile: probabilities into the P registers (bf16), the
  // reference maximum (lazy, see lazy_max) and the sum updated; returns the factor
  // the accumulator must be scaled by (exactly 1 when the reference stays).
  static __device__ __forceinline__ float softmax(const f32x16_t (&s)[KB], float c, float& m_run, float& l_run,
                                                  bf16x8_t (&pb)[KB][2]) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][r]);
    mx = pair_max<32>(mx) * c;
    const float m_new = lazy_max(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = m_new == m_run ? 1.0f : fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_use));
        psum += e;
        pb[kb][r >> 3][r & 7] = static_cast<__bf16>(e);
      }
    }
    l_run = l_run * alpha + psum;
    return alpha;
  }

  static __device__ __forceinline__ void rescale(float alpha, f32x16_t (&acc)[DB]) {
    if (__ballot(alpha != 1.0f) != 0) {
      // a real branch (the empty asm keeps the compiler from predicating the
      // rescale into every tile): most tiles leave the running maxima unchanged
      asm volatile("");
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
  }

  // O^T += V^T P^T.  The P registers of step (kb, st) hold, in MFMA k order, keys
  // 32 kb + 16 st + 4 half + {0..3} and then the same plus 8; the A operand lane
  // (32 db + col, half) needs V^T at those keys.  With the transpose read, lane l
  // of a 16-lane group receives element (l & 3) of the 4-element rows addressed
  // by lanes 4 e + l / 4 (e = 0..3), so lane s addresses key base + s / 4 at
  // d = 32 db + 16 (group & 1) + 4 (s & 3): key_off and d_off below.
  static __device__ __forceinline__ void pv(const uint16_t* lv, const bf16x8_t (&pb)[KB][2], int key_off,
                                            int d_off, f32x16_t (&acc)[DB]) {
    if constexpr (KV8) {
      // One 8-bit transpose read per product: addressing lane a (= lane % 16) of
      // group G (= lane / 16) points at key 32 kb + 16 st + key_off (key_off =
      // 8 (e / 4) + 4 half + e % 4 for e = a / 2) and at bytes 8 (a % 2) of chunk
      // 2 db + G % 2, so lane (d = 32 db + lane % 32, half) receives V at d for the 8
      // keys of its P registers, in their order.  d_off: 8 (a % 2) + chunk parity.
      const uint8_t* lvb = reinterpret_cast<const uint8_t*>(lv);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int r = 32 * kb + 16 * st + key_off;  // swz_v(r) == swz_v(key_off)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int at = r * RB + 16 * ((2 * db + (d_off & 1)) ^ swz_v(key_off)) + (d_off & 8);
            const bf16x8_t a = fp8x8_to_bf16x8(read_tr8(lvb + at));
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][st], acc[db], 0, 0, 0);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int r0 = 32 * kb + 16 * st + key_off;
        const int r1 = r0 + 8;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          // chunk (32 db + d_off) / 8 of rows r0 and r1 (swz_v(r0) == swz_v(r1) == swz_v(key_off):
          // they differ from key_off by multiples of 8)
          const int at = 8 * ((4 * db + d_off / 8) ^ swz_v(key_off)) + d_off % 8;
          const i16x4_t lo = read_tr(lv + r0 * D + at);
          const i16x4_t hi = read_tr(lv + r1 * D + at);
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][st], acc[db], 0, 0, 0);
        }
      }
    }
  }

  template <typename Emit>
  static __device__ void run(const RunParams& p, const WorkItem& it, const Variant& var, float* lds_f,
                             Emit&& emit) {
    uint16_t* lds_h = reinterpret_cast<uint16_t*>(lds_f);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31;    // query column of this lane
    const int half = lane >> 5;   // lane half: which 4-row groups of each 8
    const int g = p.group;
    const int rows_valid = it.qo_count * g;
    const int rho = wave * 32 + col;                  // folded row of this lane's column
    const bool row_ok = rho < rows_valid;
    const int t_local = rho / g;
    // addresses of the V^T operand reads (see pv): bf16, key and element offsets of
    // the 16-bit transpose read; FP8, key of this addressing lane and, packed, its
    // byte half (8 (a % 2)) and chunk parity (G % 2)
    const int a16 = lane & 15;
    const int key_off = KV8 ? 8 * ((a16 >> 1) >> 2) + 4 * (lane >> 5) + ((a16 >> 1) & 3)
                            : 4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2);
    const int d_off = KV8 ? 8 * (a16 & 1) + ((lane >> 4) & 1) : 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // variant state of this lane's row: ALiBi slope and position, tree-mask row
    const bool alibi = VAR && var.has_alibi;
    const float slope = alibi && row_ok ? var.alibi[it.kv_head * g + rho % g] : 0.0f;
    const int pos = it.q_pos + t_local;
    const uint64_t tm =
        VAR && it.tree_lo != kNoTree && row_ok ? var.tree[it.qo_begin + t_local] : ~uint64_t(0);

    // Q rows of this wavefront as the B operand: Q[rho][16 ks + 8 half + 0..7]
    bf16x8_t qreg[DK];
    {
      const uint16_t* qb = static_cast<const uint16_t*>(p.q);
      const int64_t qrow = static_cast<int64_t>(it.qo_begin + t_local) * p.h_qo + it.kv_head * g + rho % g;
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (row_ok) v = *reinterpret_cast<const u32x4_t*>(qb + qrow * D + 16 * ks + 8 * half);
        qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
      }
    }

    f32x16_t acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
    float m_run = kNegInf;   // running max (base-2 units), shared by both lane halves
    // logits in base 2 are c * s: without a soft-cap the scale is folded into the
    // exponent's fma; with one, s is first mapped to cap * tanh(s / cap) in base 2
    const float c = CAP ? 1.0f : p.scale_log2;
    float l_run = 0.0f;      // this half's share of the running sum

    const int ntok = it.kv_end - it.kv_begin;
    const int ntiles = (ntok + BC - 1) / BC;
    const __amdgpu_buffer_rsrc_t krs = row_rsrc(p.k_pool, RB);
    const __amdgpu_buffer_rsrc_t vrs = row_rsrc(p.v_pool, RB);
    const __amdgpu_buffer_rsrc_t irs = row_rsrc(p.kv_indices, 0);
    const uint32_t rpp = static_cast<uint32_t>(p.h_kv * p.page_size);
    Rows rows;
    // Two buffers: tile t lives in buffer t % 2.  The gather of tile t + 1 into the
    // other buffer and the page ids of tile t + 2 are issued before tile t is
    // computed and waited for at the next step.
    if (ntiles > 0) {
      load_rows(p, irs, it, 0, wave, lane, rows);
      gather(krs, vrs, rpp, rows, lds_addr_of(lds_h), wave, lane);
      if (ntiles > 1) load_rows(p, irs, it, 1, wave, lane, rows);
    }
    // One tile step: buffer cur holds tile t, the other one takes tile t + 1.  The
    // LDS base is made opaque per step, so the gathers' LDS addresses are formed
    // next to each load (scalar adds) instead of being computed once for the whole
    // item and held in scalar registers, which spilled them.
    auto tile = [&](int t, int cur) {
      uint32_t lbase = lds_addr_of(lds_h);
      asm volatile("" : "+s"(lbase));
      const uint16_t* lk = lds_h + cur * STAGE;
      const uint32_t nb = lbase + static_cast<uint32_t>((1 - cur) * STAGE * 2);
      // this wavefront's gather of tile t (and the ids of tile t + 1) has landed;
      // after the barrier every wavefront's has, and every wavefront is done with
      // tile t - 1, whose buffer now takes tile t + 1
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      // the gather of tile t + 1, a slice after each half block of S^T products
      const bool more = t + 1 < ntiles;
      f32x16_t s[KB];
      qk(lk, qreg, col, half, s, [&](int h) {
        constexpr int H = DK / 2;  // hook calls per tile
        if (more) gather(krs, vrs, rpp, rows, nb, wave, lane, h * NI / H, (h + 1) * NI / H);
      });
      if (t + 2 < ntiles) load_rows(p, irs, it, t + 2, wave, lane, rows);
      cap_and_mask(p, it, t, t_local, half, alibi, slope, pos, tm, s);
      bf16x8_t pb[KB][2];
      const float alpha = softmax(s, c, m_run, l_run, pb);
      rescale(alpha, acc);
      pv(lk + VOFF, pb, key_off, d_off, acc);
    };
    // tiles in pairs, so that each step's buffers sit at fixed LDS offsets (the
    // reads then take them as immediate offsets instead of per-tile address math)
    for (int t = 0; t < ntiles; t += 2) {
      tile(t, 0);
      if (t + 1 < ntiles) tile(t + 1, 1);
    }

    // result: this lane's column holds O^T[d][rho] for d = 32 db + 8 (r/4) + 4 half + r%4
    const float l_tot = pair_sum<32>(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse2 = l_tot > 0.0f ? m_run + fast_log2(l_tot) : kNegInf;
    if (row_ok) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d = 32 * db + 8 * rq + 4 * half;
          emit(rho, d, acc[db][4 * rq] * inv, acc[db][4 * rq + 1] * inv, lse2);
          emit(rho, d + 2, acc[db][4 * rq + 2] * inv, acc[db][4 * rq + 3] * inv, lse2);
        }
      }
    }
    __syncthreads();  // LDS free for the next item
  }
};

}  // namespace bsr
