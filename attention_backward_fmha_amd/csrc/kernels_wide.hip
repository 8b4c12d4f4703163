// kernels_wide.hip -- the main backward kernel in its wide layout (gfx950): eight waves per
// work group, two per SIMD, 256-key tiles, 32-row query blocks.  Serves d_qk = d_v = 128 or 64
// without a bias, with or without dropout; kernels.hip holds the four-wave layout for the other
// cases and the other stages.
#include "device.h"
#include "kernels.h"
#include "tiling.h"

namespace fmha {
namespace {

// ------------------------------------------------------------------------------------------
// Stage 2, wide layout (d_qk = d_v = D = 128 or 64, no bias).  512 threads = 8 waves, two
// per SIMD, so that one wave's matrix products overlap the other's LDS reads and exponentials
// (one wave per SIMD cannot keep more than about a quarter of the CU's LDS bandwidth busy).
// A key tile has 256 keys; wave w owns keys 32w .. 32w+31 (lane l32 holds key 32w +
// kmap(l32)), keeps its dK and dV accumulators and its V rows in registers, and reads K from
// LDS.  A step is one query block of 32 rows of one query head:
//   S = Q K_w^T, dP = dO V_w^T              A operands: Q, dO rows from LDS (16-byte reads)
//   P = exp2(S*scale*log2e - L), dS = P (dP - D)            the lane's key, 16 queries
//   dV_w += P^T dO, dK_w += dS^T Q          A from registers, B by transposing LDS reads
//   dS -> LDS (key-major: each lane writes its key's 16 queries as four 8-byte runs)
//   dQ = dS K over the tile's 256 keys      one 32x32 output tile per wave, done by the four
//                                           waves of one half, the halves taking turns; its
//                                           A operand comes from the key-major dS and its B
//                                           operand from K, both by transposing reads
// Q, dO, L, D and dS are double-buffered, so a step has one barrier: the half that computes
// the step's dQ does it at the start of the next step, while the other half already works on
// that step.  The masks are applied only to the 32 x 32 blocks that straddle a mask edge or
// the tile's last key (a wave-uniform test), and the L/D loads of the next step are selected
// where they are stored, so no wave waits on a global load inside a step.
//
// LDS banks: 64 of 4 bytes.  8-byte reads (plain or transposing) are served 32 lanes per
// cycle: the bank-conflict counter is zero for every transposing read below, each of whose
// half-waves touches every bank once, and was not for rows chosen to suit 16-lane groups.  Q,
// dO and K rows hold D bf16 + 8 of padding (kRowQ = D + 8 in the kernel: 68 dwords at D =
// 128, 36 at D = 64; either is 4 times an odd number, so row r starts at bank 4r (D = 128) or
// 4 * (9r mod 16) (D = 64) modulo 64).
//   - a transposing 8-byte read (two 16-lane groups reading the two 32-byte halves of the
//     same 4 rows) needs its 4 rows to start 16 banks apart: rows r, r + 4, r + 8, r + 12
//     modulo 16;
//   - 16-byte row reads need at least 16 rows distinct modulo 16 in each 16-lane group; the
//     row orders below were also measured free of conflicts (an order meeting only that
//     condition was not).
// Rows are therefore stored permuted inside each 32-row block by one bit permutation (qrow:
// one-to-one, linear over GF(2)) for the query rows of Q and dO and for the keys of the K
// tile.  The bits a read's lanes vary and the bits its unrolled steps vary map to disjoint row
// bits, so every LDS offset of the unrolled loops is a per-lane base plus a constant.  The
// key-major dS tile (dslot) has 72-byte rows (18 dwords): the 4 keys of a transposing read
// (key bits 0-1) go to row bits 3-4, 8 rows = 16 banks apart.  Its 8-byte writes (four per
// lane and step) still show conflicts, about 5% of the step's LDS cycles.
constexpr int kRowT = 36;    // dS^T rows (one per key): 32 bf16 + 4

__device__ __forceinline__ int bit_of(int x, int i) { return (x >> i) & 1; }

// LDS row of query row (or key) m of a step: bits m0..m4 go to r0 = m3, r1 = m2, r2 = m0,
// r3 = m1, r4 = m4.  The dV/dK products' transposing reads of lane half hi, reduction step t
// and read h take query rows 16t + 8h + 4hi + {0..3}, i.e. rows 16t + h + 2hi + 4 * {0..3};
// dQ's transposing reads take keys 16kk + 8hi + 4h + {0..3}, i.e. rows 16kk + 2h + hi +
// 4 * {0..3}.  (Row reads of S through kmap's key order also measured free of conflicts,
// where an order built only for a 16-consecutive-lane bank model was not.)
__device__ __forceinline__ int qrow(int m) {
  return (m & ~31) | bit_of(m, 3) | bit_of(m, 2) << 1 | bit_of(m, 0) << 2 | bit_of(m, 1) << 3 | bit_of(m, 4) << 4;
}

// Row of key k in the key-major dS tile: s0 = k3, s1 = k2, s2 = k4, s3 = k0, s4 = k1.  dQ's
// transposing reads take keys 16kk + 8hi + 4h + {0..3} onto rows dslot(8hi + {0..3}) +
// 32(kk / 2) + 4(kk % 2) + 2h.
__device__ __forceinline__ int dslot(int k) {
  return (k & ~31) | bit_of(k, 3) | bit_of(k, 2) << 1 | bit_of(k, 4) << 2 | bit_of(k, 0) << 3 | bit_of(k, 1) << 4;
}

// x as three bf16 parts (x = p1 + p2 + p3 to within fp32 rounding) followed by five zeros.
__device__ __forceinline__ u32x4 split3(float x) {
  const __bf16 p1 = (__bf16)x;
  const float r1 = x - (float)p1;
  const __bf16 p2 = (__bf16)r1;
  const __bf16 p3 = (__bf16)(r1 - (float)p2);
  return u32x4{__builtin_bit_cast(unsigned, bf16x2{p1, p2}), (unsigned)__builtin_bit_cast(uint16_t, p3), 0u, 0u};
}

// dS of the lane's key for the step's 32 queries into the key-major tile (row `row` =
// dslot(key)): register 4u + e holds query 8u + 4hi + e, so each u is one 8-byte write of
// four consecutive queries.
__device__ __forceinline__ void write_dst(uint16_t* dst, const float (&d)[16], int row, int hi) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
    *(u32x2*)&dst[row * kRowT + 8 * u + 4 * hi] = u32x2{pack_bf16(d[4 * u], d[4 * u + 1]), pack_bf16(d[4 * u + 2], d[4 * u + 3])};
}

template <int D, int DQM, bool XD, bool RB>
__global__ __launch_bounds__(512) void k_bwd_wide(const KParams p) {
  static_assert(D == 128 || D == 64, "head dims of the wide layout");
  constexpr int TN = 256, TM = 32, kRowQ = D + 8, NB = D / 32;  // NB: 32-column blocks
  constexpr bool DET = DQM == 1;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[TN * kRowQ];          // K tile
  __shared__ __attribute__((aligned(16))) uint16_t qo_lds[2][2][TM * kRowQ];   // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) uint16_t ds_lds[2][TN * kRowT];      // [buffer] dS^T
  // dropout: D of the step's rows per buffer (with dropout D is not folded into dP)
  __shared__ __attribute__((aligned(16))) float dd_lds[XD ? 2 * TM : 4];
  // deterministic mode with items of several key tiles (RB): the item's earlier partial of the
  // block whose dQ a wave computes next, loaded straight into LDS one step ahead (a 4 KB slot
  // for each of waves 0-3; it does not fit beside the dropout arrays at D = 128, which then load
  // it at the start of the products).  Items of one tile have nothing to read back.
  static_assert(DET || !RB, "read-back is a deterministic-mode matter");
  constexpr bool PV = RB && (D == 64 || !XD);
  __shared__ __attribute__((aligned(16))) float pv_lds[PV ? 4 * 1024 : 4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // the same value, in a scalar register
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int g16 = lane >> 4;
  const int i16 = lane & 15;

  const int nbh = p.Hkv * p.B;
  // the work group's work item: grid order, or the cost order prepare wrote
  int wid = p.order != nullptr ? p.order[blockIdx.x] : (int)blockIdx.x;
  if ((unsigned)wid >= gridDim.x) wid = (int)blockIdx.x;  // a list from another prepare: stay in range
  const int ip = wid / nbh;
  const int item = ip / p.kv_parts;
  const int part = ip - item * p.kv_parts;
  const int rem = wid - ip * nbh;
  const int g = rem % p.Hkv;
  const int b = rem / p.Hkv;
  const bool group = p.seqstart_q != nullptr;
  const Seg sg = seg_of(p, b);
  const MaskGeom mg = mask_geom(p.mask_type, p.window_left, p.window_right, sg.lq, sg.lk);
  int64_t w_lo = 1, w_hi = 0;  // query blocks already in this item's split (deterministic)
  int64_t u_lo = 1, u_hi = 0;  // union of the item's tiles' query block ranges (parts)
  for (int tsub = 0; tsub < p.tiles_per_item; ++tsub) {
    const int j = item * p.tiles_per_item + tsub;
    if ((int64_t)j * TN >= sg.lk) break;
    int64_t lo, hi2;
    qblocks_for_tile(mg, sg.lq, sg.lk, j, TM, TN, &lo, &hi2);
    if (hi2 >= lo) {
      const bool had = u_hi >= u_lo;
      u_lo = had ? min(u_lo, lo) : lo;
      u_hi = had ? max(u_hi, hi2) : hi2;
    }
  }
  const int64_t nbu = u_hi >= u_lo ? u_hi - u_lo + 1 : 0;
  const int64_t nu = nbu * p.group_size;
  const int64_t u_a = nu * part / p.kv_parts;
  const int64_t u_e = nu * (part + 1) / p.kv_parts;

  const int tr_row = i16 >> 2;                        // row inside a 4-row transposing read
  const int tr_col = 16 * (g16 & 1) + 4 * (i16 & 3);  // its columns inside a 32-column tile
  const int key_w = 32 * wave + kmap(l32);            // the lane's key inside the tile
  // LDS row of the lane's transposing reads of Q and dO (reduction step 0; +16 for step 1,
  // +1 for the second read): query row 4hi + tr_row
  const int tq_row = qrow(4 * hi + tr_row);
  // K and dS rows of the lane's transposing reads for dQ: key 8hi + tr_row of reduction step 0
  const int tk_row = qrow(8 * hi + tr_row), td_row = dslot(8 * hi + tr_row);
  const int q_row = qrow(l32);                        // LDS row of the lane's query (S, dP)
  const float inv_c = 1.f / p.scale_log2;
  // B operand of ones in reduction slots 0..2 of lane half 0 (bf16 1.0 = 0x3F80), zeros in
  // half 1: the product with a padding chunk adds its three parts
  // (at D = 128 it is built where it is used instead, from a lane index read there, so that
  // it does not take four registers across the step loop)
  const bf16x8 ones3_kept = __builtin_bit_cast(bf16x8, u32x4{hi ? 0u : 0x3F803F80u, hi ? 0u : 0x3F80u, 0u, 0u});
  const int qs1 = (int)p.q_s[1];
  const int os1 = (int)p.do_s[1];

  for (int tsub = 0; tsub < p.tiles_per_item; ++tsub) {
    const int j = item * p.tiles_per_item + tsub;
    const int64_t key0 = (int64_t)j * TN;
    if (key0 >= sg.lk) break;
    if (tsub > 0) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // every wave is done with the previous tile's LDS
    }
    const int nk = (int)min((int64_t)TN, sg.lk - key0);
    int64_t qb_lo, qb_hi;
    qblocks_for_tile(mg, sg.lq, sg.lk, j, TM, TN, &qb_lo, &qb_hi);
    const int nblk = qb_hi >= qb_lo ? (int)(qb_hi - qb_lo + 1) : 0;
    const int64_t lo64 = mg.left >= 0 ? mg.delta - mg.left : -sg.lq;
    const int64_t hi64 = mg.right >= 0 ? mg.delta + mg.right : sg.lk;
    const int lo_d = (int)max(lo64, -sg.lq);
    const int hi_d = (int)min(hi64, sg.lk);
    const unsigned span = (unsigned)(hi_d - lo_d);

    // ---- prologue.  The tile's loads are all issued before the first wait: the K tile (D / 16
    // chunks per thread, into registers), then step n0's Q and dO rows (below), then the wave's
    // V rows (the B operand of dP, kept in registers); the K chunks and the first step's rows
    // then go to LDS.  (Loads and LDS writes taken one chunk at a time cost one HBM round trip
    // per chunk, about 25k cycles per tile.)
    const int ln_t = lane_here();
    const int tid_t = 64 * wave_s + ln_t;
    u32x4 kx[D / 16];
    {
      const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(
          p.k + elem_off(p.k_s, group, b, sg.k_row0 + key0, g), (uint32_t)((nk - 1) * (int)p.k_s[1] + D) * 2u);
      const int ks1 = (int)p.k_s[1];
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        const int id = tid_t + 512 * i;
        const int kr = id / (D / 8), c = id % (D / 8);
        kx[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, (kr * ks1 + c * 8) * 2, 0, 0);
      }
    }
    bf16x8 vw[D / 16];
    const auto load_v = [&]() {
      const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(
          p.v + elem_off(p.v_s, group, b, sg.k_row0 + key0, g), (uint32_t)((nk - 1) * (int)p.v_s[1] + D) * 2u);
      const int vs1 = (int)p.v_s[1];
      const int kv = 32 * wave_s + kmap(ln_t & 31);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        vw[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, (kv * vs1 + 16 * kk + 8 * (ln_t >> 5)) * 2, 0, 0));
    };
    const auto store_k = [&]() {
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        const int id = tid_t + 512 * i;
        const int kr = id / (D / 8), c = id % (D / 8);
        *(u32x4*)&k_lds[qrow(kr) * kRowQ + c * 8] = kx[i];
      }
    };
    f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
    for (int n = 0; n < D / 32; ++n) {
      dk_acc[n] = f32x16{};
      dv_acc[n] = f32x16{};
    }

    // steps of this part: as in k_bwd_main
    const auto steps_before = [&](int64_t u) -> int {
      if (nbu == 0) return 0;
      const int64_t c = min(max(u_lo + u % nbu - qb_lo, (int64_t)0), (int64_t)nblk);
      return (int)((u / nbu) * nblk + c);
    };
    const int n0 = steps_before(u_a);
    const int n1 = steps_before(u_e);

    // ---- step cursors.  The work group's steps [n0, n1) number (query head, query block)
    // pairs head-major and are taken last to first: query blocks in descending order.  Work
    // groups go to the 8 XCDs round robin, so with Hkv * B a multiple of 8 the items of one
    // (segment, K/V head) share an XCD, and those started together then read the same Q and
    // dO blocks at about the same time, from its L2 (in ascending order their first blocks
    // differ by item).  Causal 2 x 32 x 4096: 11% fewer HBM bytes read.  A cursor holds a
    // step's count, query head and first row.
    // Buffer resources span one query head's rows of the segment and a step's rows go into the
    // per-lane offset, so rows past the segment end read as zeros and stores or atomics to them
    // are dropped; a resource is rebuilt only when the head changes ----
    struct Cur {
      int n, h, r;
    };
    const int row_lo = (int)qb_lo * TM, row_hi = (int)qb_hi * TM;
    const int lq = (int)sg.lq;
    auto advance = [&](Cur& c) {
      ++c.n;
      c.r -= TM;
      if (c.r < row_lo) {
        c.r = row_hi;
        --c.h;
      }
    };
    const uint32_t q_bytes = lq > 0 ? (uint32_t)((lq - 1) * qs1 + D) * 2u : 0u;
    const uint32_t o_bytes = lq > 0 ? (uint32_t)((lq - 1) * os1 + D) * 2u : 0u;
    Cur pc;  // the step being prefetched
    pc.n = n0;
    const int m_first = n1 > n0 ? n1 - 1 : n0;
    pc.h = g * p.group_size + (nblk > 0 ? m_first / nblk : 0);
    pc.r = row_lo + (nblk > 0 ? m_first % nblk : 0) * TM;
    __amdgpu_buffer_rsrc_t rq, ro, rl, rd;
    auto head_rsrc = [&](int hh) {
      rq = buffer_rsrc(p.q + elem_off(p.q_s, group, b, sg.q_row0, hh), q_bytes);
      ro = buffer_rsrc(p.dout + elem_off(p.do_s, group, b, sg.q_row0, hh), o_bytes);
      const int64_t w0 = (int64_t)hh * p.rows_q + sg.ws_row0;
      rl = buffer_rsrc(p.lse2 + w0, (uint32_t)lq * 4u);
      rd = buffer_rsrc(p.dsum + w0, (uint32_t)lq * 4u);
    };
    head_rsrc(pc.h);

    // ---- staging.  D = 128: thread t loads 16 bytes of Q and of dO (row t/16, chunk t%16);
    // D = 64: waves 0-3 load Q and waves 4-7 dO, 16 bytes per thread (row (t%256)/8, chunk
    // t%8).  Wave 0 loads L (lanes 0..31) and D (lanes 32..63) ----
    u32x4 q_pre, o_pre;
    float l_pre = 0.f, d_pre = 0.f;  // wave 0: L (lanes 0..31) and D (lanes 32..63) loads in flight
    int nq_pre = 0;
    const bool st_o = D == 64 && wave_s >= 4;  // D = 64: this wave stages dO
    const int st_row = D == 128 ? tid >> 4 : (tid & 255) >> 3, st_c = tid & (D / 8 - 1);
    const int st_lds = qrow(st_row) * kRowQ + st_c * 8;
    const int q_lane = (st_row * (st_o ? os1 : qs1) + st_c * 8) * 2, o_lane = (st_row * os1 + st_c * 8) * 2;
    auto load_step = [&]() {  // the prefetch cursor's step, then advance it
      const bool valid = pc.n < n1;
      const __amdgpu_buffer_rsrc_t none = buffer_rsrc(p.q, 0u);
      nq_pre = valid ? min(TM, lq - pc.r) : 0;
      if constexpr (D == 128) {
        q_pre = __builtin_amdgcn_raw_buffer_load_b128(valid ? rq : none, q_lane + pc.r * qs1 * 2, 0, 0);
        o_pre = __builtin_amdgcn_raw_buffer_load_b128(valid ? ro : none, o_lane + pc.r * os1 * 2, 0, 0);
      } else {
        // a branch on the wave-uniform flag, so that each load takes one scalar resource
        if (st_o)
          q_pre = __builtin_amdgcn_raw_buffer_load_b128(valid ? ro : none, q_lane + pc.r * os1 * 2, 0, 0);
        else
          q_pre = __builtin_amdgcn_raw_buffer_load_b128(valid ? rq : none, q_lane + pc.r * qs1 * 2, 0, 0);
      }
      if (wave == 0) {  // two loads with wave-uniform resources
        const float lv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(valid ? rl : none, (pc.r + l32) * 4, 0, 0));
        const float dv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(valid ? rd : none, (pc.r + l32) * 4, 0, 0));
        l_pre = lv;  // selected where they are stored, so nothing waits for the loads here
        d_pre = dv;
      }
      const int h_old = pc.h;
      advance(pc);
      if (pc.h != h_old && pc.n < n1) head_rsrc(pc.h);
    };
    auto store_step = [&](int buf) {
      if constexpr (D == 128) {
        *(u32x4*)&qo_lds[buf][0][st_lds] = q_pre;
        *(u32x4*)&qo_lds[buf][1][st_lds] = o_pre;
      } else {
        *(u32x4*)&qo_lds[buf][st_o ? 1 : 0][st_lds] = q_pre;
      }
      // the padding columns of Q row r carry -L2[r]/c, those of dO row r carry -D[r] (three
      // bf16 parts each); a row past the segment end gets -1e30, so its P is exactly 0.  With
      // dropout the dO padding is 0 and D goes to dd_lds: dS = P (Z dP - D) needs dP alone
      if (wave == 0) {
        const float x = lane < 32 ? (l32 < nq_pre ? -l_pre * inv_c : -1e30f) : (XD ? 0.f : -d_pre);
        *(u32x4*)&qo_lds[buf][hi][q_row * kRowQ + D] = split3(x);
        if (XD && lane >= 32) dd_lds[buf * TM + l32] = d_pre;
      }
    };

    // ---- dQ of a finished step from ds_lds[buf]: this wave's 32 columns ----
    // accumulator resources of one query head (rebuilt when the head changes)
    auto dq_rsrc = [&](int hh) -> __amdgpu_buffer_rsrc_t {
      if (DET)
        return buffer_rsrc(p.dq_acc + (int64_t)item * p.split_stride + (int64_t)hh * p.head_stride +
                               sg.acc_row0 * D, (uint32_t)(row_hi + TM) * D * 4u);
      if (DQM == 2)
        return buffer_rsrc((const uint16_t*)p.dq_acc + (int64_t)b * p.split_stride + (int64_t)hh * p.head_stride,
                           (uint32_t)(row_hi + TM) * D * 2u);
      return buffer_rsrc(p.dq_acc + (int64_t)hh * p.head_stride + sg.acc_row0 * D, (uint32_t)lq * D * 4u);
    };
    const int nd = wave & (NB - 1);  // this wave's 32 dQ columns
    // the waves that compute the dQ of the work group's step s: among waves 0-3, the older
    // wave of each SIMD, which wins issue arbitration and would otherwise wait longest at the
    // barrier (measured 1-2% faster than spreading dQ over all eight waves in turn): D = 128,
    // all four (one 32-column tile each); D = 64, waves 0-1 and 2-3 taking turns
    auto dq_turn = [&](int s) { return D == 128 ? wave_s < 4 : (wave_s >> 1) == (s & 1); };
    auto dq_step = [&](int buf, const __amdgpu_buffer_rsrc_t& rdq, int r) {
      // deterministic mode: the partial an earlier tile of the item left for this block, from
      // the wave's LDS slot (loaded a step ahead, below) or read back first, so that the
      // products below hide the load latency
      u32x4 prev[4] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
      if constexpr (PV) {
#pragma unroll
        for (int u = 0; u < 4; ++u) prev[u] = *(const u32x4*)&pv_lds[(wave_s & 3) * 1024 + u * 256 + lane * 4];
      } else if constexpr (RB) {
        const int qbn = r / TM;
        const __amdgpu_buffer_rsrc_t rprev = qbn >= w_lo && qbn <= w_hi ? rdq : buffer_rsrc(p.dq_acc, 0u);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          prev[u] = __builtin_amdgcn_raw_buffer_load_b128(rprev, (r * D + nd * 1024 + u * 256 + lane * 4) * 4, 0, kPartialPolicy);
      }
      f32x16 acc = f32x16{};
      // A operand: keys 16kk + 8hi + {0..3, 4..7} of query l32, two transposing reads of the
      // key-major dS; B operand: the same keys' rows of K, columns 32nd .. 32nd + 31
      const uint16_t* dsb = &ds_lds[buf][td_row * kRowT + tr_col];
      const uint16_t* kt = &k_lds[tk_row * kRowQ + 32 * nd + tr_col];
      // operands of reduction step kk: dS row chunk and the transposed K block; loaded two
      // steps ahead of their product (the fences keep that order)
      bf16x8 da[2], bk[2];
      auto ld = [&](int kk) {
        const int db = (32 * (kk >> 1) + 4 * (kk & 1)) * kRowT;
        const int kb = 16 * kk * kRowQ;
        da[kk & 1] = tr_read(&dsb[db], &dsb[db + 2 * kRowT]);
        bk[kk & 1] = tr_read(&kt[kb], &kt[kb + 2 * kRowQ]);
      };
      ld(0);
      ld(1);
#pragma unroll
      for (int kk = 0; kk < TN / 16; ++kk) {
        acc = mfma(da[kk & 1], bk[kk & 1], acc);
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 2 < TN / 16) ld(kk + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (DET) {
        const int voff = (r * D + nd * 1024 + lane * 4) * 4;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          __builtin_amdgcn_raw_buffer_store_b128(
              u32x4{__float_as_uint(__uint_as_float(prev[u][0]) + acc[4 * u]),
                    __float_as_uint(__uint_as_float(prev[u][1]) + acc[4 * u + 1]),
                    __float_as_uint(__uint_as_float(prev[u][2]) + acc[4 * u + 2]),
                    __float_as_uint(__uint_as_float(prev[u][3]) + acc[4 * u + 3])},
              rdq, voff + 1024 * u, 0, kPartialPolicy);
      } else if (DQM == 2) {
        // packed bf16 adds: lanes 2c and 2c+1 trade their (row k, row 8+k) words so that each
        // holds one row of columns 2c, 2c+1; the block is stored tile by tile (tile nd at
        // 2048 bytes * nd), register pair k2 at 256 * k2, lane l's word at 4 * l
        const bool odd = (lane & 1) != 0;
        const unsigned sel = odd ? 0x03020706u : 0x05040100u;
        const int vbase = r * D * 2 + nd * 2048 + lane * 4;
#pragma unroll
        for (int k2 = 0; k2 < 8; ++k2) {
          const unsigned mine = pack_bf16(acc[k2], acc[8 + k2]);
          const unsigned other = xor1(mine);
          const unsigned v = __builtin_amdgcn_perm(other, mine, sel);
          asm volatile("buffer_atomic_pk_add_bf16 %0, %1, %2, 0 offen offset:%3" ::"v"(v), "v"(vbase), "s"(rdq),
                       "n"(k2 * 256));
        }
      } else {
        // register rr holds row 8(rr/4) + 4hi + rr%4, column 32nd + l32
        const int voff = ((r + 4 * hi) * D + 32 * nd + l32) * 4;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[rr], rdq, voff + (8 * (rr >> 2) + (rr & 3)) * D * 4, 0, 0);
      }
    };

    Cur cc = pc;  // the step being computed
    if (n1 > n0) load_step();
    load_v();
    store_k();
    if (n1 > n0) {
      store_step(0);
      load_step();
    }
    __syncthreads();
    Cur dc = cc;  // the step whose dQ is pending (the previous one)
    __amdgpu_buffer_rsrc_t rdq = dq_rsrc(dc.h);
    const bool key_ok = key_w < nk;
    for (int n = n0; n < n1; ++n) {
      const int buf = (n - n0) & 1;
      // the pending dQ of step n-1, by the half whose turn it is
      if (n > n0 && dq_turn(n - 1 - n0)) dq_step(buf ^ 1, rdq, dc.r);
      // the wave that computes step n's dQ (in the next iteration) loads the item's earlier
      // partial of step n's block into its slot now: direct-to-LDS loads, 16 bytes per lane,
      // lane l's at 16l of each kilobyte (a block the item has not written reads as zeros)
      if constexpr (PV) {
        if (dq_turn(n - n0)) {
          // (a copy of the cursor's row: with the cursor field itself in the offset operand, the
          // host pass of this compiler left the kernel's launch stub undefined)
          const int r_pv = cc.r;
          const int qbn = r_pv / TM;
          const __amdgpu_buffer_rsrc_t rpv = qbn >= w_lo && qbn <= w_hi ? dq_rsrc(cc.h) : buffer_rsrc(p.dq_acc, 0u);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rpv, (__attribute__((address_space(3))) void*)&pv_lds[(wave_s & 3) * 1024 + u * 256], 16,
                (r_pv * D + nd * 1024 + u * 256) * 4 + lane * 16, 0, 0, kPartialPolicy);
        }
      }
      const int q0 = cc.r;
      // ---- S, dP, P, dS, dV, dK of step n ----
      {
        float ds32[16];
        const uint16_t* qb = qo_lds[buf][0];
        const uint16_t* ob = qo_lds[buf][1];
        // S and dP, interleaved; the scheduling groups keep the LDS reads two reduction steps
        // ahead of the products that use them
        f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
        const uint16_t* qrw = &qb[q_row * kRowQ + 8 * hi];
        const uint16_t* orw = &ob[q_row * kRowQ + 8 * hi];
        const uint16_t* krw = &k_lds[qrow(key_w) * kRowQ + 8 * hi];
        // S and dP interleaved; operands loaded two reduction steps ahead of their products.
        // A ninth step multiplies the padding chunk of the Q and dO rows by ones3, which adds
        // -L2/c to S and -D to dP: then P = exp2(c S) and dS = P dP directly.
        bf16x8 qa[2], kb2[2], oa[2];
        auto ld = [&](int kk) {
          if (kk < D / 16) {
            qa[kk & 1] = *(const bf16x8*)&qrw[16 * kk];
            kb2[kk & 1] = *(const bf16x8*)&krw[16 * kk];
            oa[kk & 1] = *(const bf16x8*)&orw[16 * kk];
          } else {
            qa[kk & 1] = *(const bf16x8*)&qb[q_row * kRowQ + D];
            oa[kk & 1] = *(const bf16x8*)&ob[q_row * kRowQ + D];
          }
        };
        ld(0);
        ld(1);
        bf16x8 ones3 = ones3_kept;
#pragma unroll
        for (int kk = 0; kk <= D / 16; ++kk) {
          if (D == 128 && kk == D / 16) {
            const bool h0 = lane_here() < 32;
            ones3 = __builtin_bit_cast(bf16x8, u32x4{h0 ? 0x3F803F80u : 0u, h0 ? 0x3F80u : 0u, 0u, 0u});
          }
          s_acc = mfma(qa[kk & 1], kk < D / 16 ? kb2[kk & 1] : ones3, s_acc);
          dp_acc = mfma(oa[kk & 1], kk < D / 16 ? vw[kk] : ones3, dp_acc);
          __builtin_amdgcn_sched_barrier(0);
          if (kk + 2 <= D / 16) ld(kk + 2);
          __builtin_amdgcn_sched_barrier(0);
        }
        // P = exp2(c S), 0 for masked pairs; dS = P dP.  The mask is applied only when some
        // (key, query) pair of the wave's 32 x 32 block is outside it (the block straddles
        // the mask's edge or the tile's last key): a wave-uniform test per step
        bf16x8 pa[2], sa[2];
        // dropout: row group c (rows 8c + 4hi + e) of the lane's key takes byte (key % 4) of
        // word e of the Philox output for (key / 4, row / 4).  The four lanes of a key quad
        // (l, l^1, l^16, l^17: key bits 0-1 are lane bits 4 and 0) need the same four outputs;
        // each computes the one of its position t in the quad, transposes it to per-key words
        // of 4 row bytes, and the quad trades them
        unsigned zw[4] = {0u, 0u, 0u, 0u};
        if constexpr (XD) {
          // at D = 128 the lane values come from a lane index read here, so that they do not
          // stay live across the step loop (which spilled registers reloaded in every step)
          const int ln = D == 128 ? lane_here() : lane;
          const unsigned kpos = (unsigned)(key0 + 32 * wave_s + kmap(ln & 31));
          const unsigned t = (unsigned)(ln & 1) | ((unsigned)(ln >> 4) & 1u) << 1;
          unsigned w[4] = {kpos >> 2, (unsigned)(q0 + 8 * (int)t + 4 * (ln >> 5)) >> 2,
                           (unsigned)(b * p.Hq + cc.h), p.offset_lo};
          // the key enters each step through an empty asm statement, so that the compiler
          // derives the round keys in the step (two scalar adds per round) instead of keeping
          // all twenty live across the loop, which spilled scalar registers
          unsigned k0 = p.seed_lo, k1 = p.seed_hi;
          asm volatile("" : "+s"(k0), "+s"(k1));
          philox4x32_10(w, k0, k1);
          unsigned tw[4];
          byte_transpose4(w, tw);  // tw[k]: the 4 row bytes of key k % 4
          unsigned rr[4];
          rr[0] = sel4(tw, ((t >> 1) & 1u) | ((t & 1u) << 1));
          {
            const unsigned pu = t ^ 1u;
            rr[1] = xor1(sel4(tw, ((pu >> 1) & 1u) | ((pu & 1u) << 1)));
          }
          {
            const unsigned pu = t ^ 2u;
            rr[2] = xor16(sel4(tw, ((pu >> 1) & 1u) | ((pu & 1u) << 1)), ln);
          }
          {
            const unsigned pu = t ^ 3u;
            rr[3] = xor16(xor1(sel4(tw, ((pu >> 1) & 1u) | ((pu & 1u) << 1))), ln);
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) zw[c] = sel4(rr, t ^ (unsigned)c);
        }
        {
#pragma unroll
          for (int r = 0; r < 16; ++r) ds32[r] = __builtin_amdgcn_exp2f(s_acc[r] * p.scale_log2);
          const int dmin = (int)key0 + 32 * wave_s - q0 - (TM - 1) - lo_d;  // min over the block of key - query - lo_d
          const bool full = 32 * wave_s + 32 <= nk && dmin >= 0 && dmin + 62 <= (int)span;
          if (!full) {
            const int t0 = key_ok ? (int)key0 - q0 + key_w - lo_d - 4 * hi : (int)span + TM + 1;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                ds32[4 * c + e] = (unsigned)(t0 - (8 * c + e)) <= span ? ds32[4 * c + e] : 0.f;
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            f32x4 d4 = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (XD) d4 = *(const f32x4*)&dd_lds[buf * TM + 8 * c + 4 * hi];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * c + e;
              const float pv = ds32[r];
              // with dropout Z = 256/k where the element's byte is below k, else 0
              const float zf = XD ? (((zw[c] >> (8 * e)) & 0xFFu) < (unsigned)p.drop_k ? p.drop_scale : 0.f) : 1.f;
              const float dsv = XD ? pv * (dp_acc[r] * zf - d4[e]) : pv * dp_acc[r];
              // reduction slot of (c, e) in step c/2: read c % 2, row e of the transposing reads
              const int slot = 4 * (c & 1) + e;
              pa[c >> 1][slot] = (__bf16)(XD ? pv * zf : pv);
              sa[c >> 1][slot] = (__bf16)dsv;
              ds32[r] = dsv;
            }
          }
        }
        // dV += P^T dO, dK += dS^T Q: reduction step t covers queries 16t .. 16t + 15; lane
        // half hi takes query rows 16t + 4hi + {0..3} and then + 8.  Operand pairs are loaded
        // two products ahead; the dS write runs under the first products.
        bf16x8 bo[2], bq[2];
        // per-lane bases; each read adds a constant, which becomes the instruction's offset
        const uint16_t* obl = &ob[tq_row * kRowQ + tr_col];
        const uint16_t* qbl = &qb[tq_row * kRowQ + tr_col];
        auto ldv = [&](int i) {
          const int t = i / NB, n2 = i % NB;
          const int off = 16 * t * kRowQ + 32 * n2;
          bo[i & 1] = tr_read(obl + off, obl + off + kRowQ);
          bq[i & 1] = tr_read(qbl + off, qbl + off + kRowQ);
        };
        ldv(0);
        ldv(1);
#pragma unroll
        for (int i = 0; i < 2 * NB; ++i) {
          dv_acc[i % NB] = mfma(pa[i / NB], bo[i & 1], dv_acc[i % NB]);
          dk_acc[i % NB] = mfma(sa[i / NB], bq[i & 1], dk_acc[i % NB]);
          __builtin_amdgcn_sched_barrier(0);
          if (i + 2 < 2 * NB) ldv(i + 2);
          if (i == 0) write_dst(ds_lds[buf], ds32, dslot(key_w), hi);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      store_step(buf ^ 1);  // step n+1's tiles (zeros after the last step)
      if (dc.h != cc.h) rdq = dq_rsrc(cc.h);
      dc = cc;
      advance(cc);
      __syncthreads();  // step n's dS and step n+1's tiles are complete
      load_step();
    }
    // the last step's dQ
    if (n1 > n0 && dq_turn(n1 - 1 - n0)) dq_step((n1 - 1 - n0) & 1, rdq, dc.r);

    // ---- epilogue: dK = scale * dK_acc, dV = dV_acc as bf16, or this part's fp32 partials.
    // Each lane holds one column of 16 keys, so the values go through LDS: the wave writes a
    // pass (2D bytes per key: all of dK or dV in bf16, or D/2 fp32 columns of a partial) into
    // its 32 rows of the K tile, row m for the key of M index m, and reads it back in 16-byte
    // chunks, 16 lanes per row, so that each buffer store covers four keys' contiguous runs.
    // The stores' resources span the tile's nk rows, so the range check drops keys past the
    // tile end.
    __syncthreads();  // the last dQ products have read the K tile
    {
      constexpr int kChunks = D / 8;  // 16-byte chunks per row and pass
      // the lane index again, from mbcnt: per-lane values derived here are not merged with the
      // ones computed before the step loop, so they do not stay live (and spill) across it
      const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      uint16_t* ep = &k_lds[32 * wave_s * kRowQ];
      // write: lane (l32, hi) holds M indices 8c + 4hi + e; read: lane l takes row 4i + l / 16
      // (i = 0 .. 32 * kChunks / 64 - 1), chunk l % 16 (D = 128) or rows 8i + l / 8, chunk l % 8
      uint16_t* ep_w = ep + 4 * (ln >> 5) * kRowQ + (ln & 31);
      constexpr int kRowsPerRead = 64 / kChunks;
      const int rd_row = ln / kChunks, rd_c = ln % kChunks;
      const uint16_t* ep_r = ep + rd_row * kRowQ + 8 * rd_c;
      // key of read row kRowsPerRead * i + rd_row: kmap is linear, key = kmap(rd_row) + kmap(kRowsPerRead * i)
      const int kl_lane = wave_s * 32 + kmap(rd_row);
      const auto pass = [&](const int ps, const bool part_out) {
        const bool is_v = part_out ? ps >= 2 : ps == 1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int mo = (8 * (r >> 2) + (r & 3)) * kRowQ;
          if (!part_out) {
#pragma unroll
            for (int n = 0; n < NB; ++n) ep_w[mo + 32 * n] = to_bf16_bits(is_v ? dv_acc[n][r] : dk_acc[n][r] * p.scale);
          } else {
#pragma unroll
            for (int n2 = 0; n2 < NB / 2; ++n2) {
              const int n = (ps & 1) * (NB / 2) + n2;
              *(float*)&ep[(4 * (ln >> 5) * kRowQ + mo) + 2 * (32 * n2 + (ln & 31))] = is_v ? dv_acc[n][r] : dk_acc[n][r];
            }
          }
        }
        __amdgpu_buffer_rsrc_t rs;
        int row_bytes, col_bytes;
        if (!part_out) {
          const int64_t* st = is_v ? p.dv_s : p.dk_s;
          uint16_t* base = (is_v ? p.dv : p.dk) + elem_off(st, group, b, sg.k_row0 + key0, g);
          row_bytes = (int)st[1] * 2;
          col_bytes = 0;
          rs = buffer_rsrc(base, (uint32_t)((nk - 1) * (int)st[1] + D) * 2u);
        } else {
          float* base = p.dkv_acc + (((int64_t)part * p.Hkv + g) * p.rows_k + sg.kws_row0 + key0) * (2 * D);
          row_bytes = 2 * D * 4;
          col_bytes = ((is_v ? D : 0) + (ps & 1) * (D / 2)) * 4;
          rs = buffer_rsrc(base, (uint32_t)nk * (uint32_t)row_bytes);
        }
        const int voff = kl_lane * row_bytes + col_bytes + 16 * rd_c;
#pragma unroll
        for (int i = 0; i < 32 * kChunks / 64; ++i) {
          const u32x4 x = *(const u32x4*)&ep_r[kRowsPerRead * i * kRowQ];
          if (part_out)
            __builtin_amdgcn_raw_buffer_store_b128(x, rs, voff + kmap(kRowsPerRead * i) * row_bytes, 0, kPartialPolicy);
          else
            __builtin_amdgcn_raw_buffer_store_b128(x, rs, voff + kmap(kRowsPerRead * i) * row_bytes, 0, 0);
        }
      };
      if (p.kv_parts == 1) {
        pass(0, false);
        pass(1, false);
      } else {
        pass(0, true);
        pass(1, true);
        pass(2, true);
        pass(3, true);
      }
    }
    if (nblk > 0) {
      const bool had = w_hi >= w_lo;
      w_lo = had ? min(w_lo, qb_lo) : qb_lo;
      w_hi = had ? max(w_hi, qb_hi) : qb_hi;
    }
  }  // tiles of the item
}

template <int D, bool XD>
void launch_wide_t(int mode, bool read_back, const KParams& kp, dim3 grid, hipStream_t stream) {
  if (mode == 1 && read_back) hipLaunchKernelGGL((k_bwd_wide<D, 1, XD, true>), grid, dim3(512), 0, stream, kp);
  else if (mode == 1) hipLaunchKernelGGL((k_bwd_wide<D, 1, XD, false>), grid, dim3(512), 0, stream, kp);
  else if (mode == 2) hipLaunchKernelGGL((k_bwd_wide<D, 2, XD, false>), grid, dim3(512), 0, stream, kp);
  else hipLaunchKernelGGL((k_bwd_wide<D, 0, XD, false>), grid, dim3(512), 0, stream, kp);
}

}  // namespace

hipError_t launch_main_wide(const Plan& plan, const KParams& kp, dim3 grid, hipStream_t stream) {
  const int mode = plan.deterministic ? 1 : (plan.dq_bf16 ? 2 : 0);
  const bool drop = plan.drop_k < 256;
  const bool rb = plan.tiles_per_item > 1;  // an item's later tiles add to its earlier partials
  if (plan.d_qk == 64) {
    if (drop) launch_wide_t<64, true>(mode, rb, kp, grid, stream);
    else launch_wide_t<64, false>(mode, rb, kp, grid, stream);
  } else {
    if (drop) launch_wide_t<128, true>(mode, rb, kp, grid, stream);
    else launch_wide_t<128, false>(mode, rb, kp, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace fmha
