// fa_fwd_mfma16.hip -- FlashAttention forward for gfx950 (CDNA4, MI355X) with 16-bit
// inputs: bf16 or fp16 (the element type E), fp32 accumulation, output in E.
//
// One workgroup (4 waves) owns 128 query rows of one (batch, query head) and
// walks the key tiles of its K/V head in order: query blocks outer, key blocks
// inner (kbwen.com FlashAttention feed, "More than two blocks").  Each wave owns
// 32 query rows; two workgroups share a CU, so two waves share each SIMD and one
// wave's exponentials overlap the other's matrix products.
//
// Per key tile of BN keys, for each wave:
//   S^T = K_tile Q_w^T          v_mfma_f32_32x32x16_{bf16,f16}, fp32 accumulate
//   -inf where masked           only on tiles that cross the diagonal or the N tail
//   mx  = rowmax S^T * c        c = scale * log2(e); one lane-half swap per row
//   if mx > m + 8: m' = mx, a = exp2(m - m'), l *= a, O *= a      (lazy rescale)
//   P   = exp2(S^T * c - m)     one FMA and one v_exp_f32 per score
//   l  += rowsum P,  O^T += V_tile^T P^T        (P rounded to E)
// and after the last tile O = O^T / l, LSE = (m + log2 l) * ln 2.
//
// This is the update the pages derive (mbrenndoerfer.com "Online Softmax
// Computation", its update equations and five steps; spicyshark.co online-softmax
// lesson, "The idea", "From softmax to attention" and "The implementation") in
// base 2, with one liberty the mathematics allows: the reference m is moved only
// when the row maximum has grown by more than 2^8.  Between moves l and O are
// both measured against the same, slightly stale m, so every term carries the
// same factor and u / l is unchanged; P stays below 2^8, far from any overflow.
// A row whose tiles so far held no finite score keeps m = -inf and adds nothing
// (the pages' guard for a fully masked block).  l sums P in fp32, before P is
// rounded to E for the PV product.
//
// Why the scores are transposed: lane L of a 32x32 MFMA output holds one column.
// With K as the A operand that column is one query row, so the row max and sum
// are in-lane except for one exchange between lane halves, and the rounded P is
// already the B operand of the PV product: P never goes through LDS.
//
// LDS, double-buffered: K and V tiles, both row-major [BN][D] with 16-byte chunks
// XOR-swizzled per row, filled straight from HBM by buffer_load_dwordx4 ... lds
// (rows past N read as zero: the buffer range ends at the last key).  The PV A
// operand (V^T) comes from ds_read_b64_tr_b16, which transposes 4 keys x 16 dims
// across each group of 16 lanes, so V needs no transposition anywhere.  The four
// tile buffers are separate arrays and the key loop is unrolled by two, so every
// access names its buffer statically: the compiler can then see that reading
// one buffer does not wait for the loads still landing in the other.
//
// Split mode (SPLIT = true) computes the same state over one contiguous range of
// keys per workgroup and writes it normalised, o = u / l and lse = m + ln l, in
// float: the partial state of the pages' merge (kbwen.com feed, "Two blocks";
// spicyshark.co lesson, "From softmax to attention", two workers).  The queries
// are then the last N of Nk positions (query i at key position i + Nk - N), a
// row with no visible key in the range gets the empty state (o = 0, lse = -inf),
// and because that offset is arbitrary a wave's diagonal may straddle two key
// tiles, so causal split kernels also check the mask on tiles before the last.
#include "fa_kernels.h"
#include "fa_mfma16_common.h"

#include <float.h>
#include <stdint.h>

namespace fa {

template <typename E, int D, int BM, int BN, bool CAUSAL, bool SPLIT>
__global__ void __launch_bounds__(BM * 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd16_kernel(const FwdParams p)
{
    typedef typename Elem<E>::x8 ex8;
    typedef typename Elem<E>::x4 ex4;
    typedef typename Elem<E>::x2 ex2;
    static_assert(BM == 128, "four waves of 32 query rows");
    static_assert(D == 64 || D == 128, "head dimension");
    static_assert(BN % 32 == 0, "key tile");
    constexpr int NW = BM / 32;
    constexpr int ROWB = D * 2;                 // bytes per K/V row
    constexpr int TILEB = BN * ROWB;            // bytes per K or V tile
    constexpr int LOADS = TILEB / 1024;         // 1 KiB wave-loads per tile (each of K, V)
    constexpr int DK = D / 16;                  // k-steps of the score product
    constexpr int ST = BN / 32;                 // 32-key score tiles per key tile
    constexpr int DT = D / 32;                  // 32-dim output tiles
    static_assert(LOADS % NW == 0, "tile loads must split evenly over the waves");

    __shared__ __attribute__((aligned(1024))) char k_lds0[TILEB];
    __shared__ __attribute__((aligned(1024))) char k_lds1[TILEB];
    __shared__ __attribute__((aligned(1024))) char v_lds0[TILEB];
    __shared__ __attribute__((aligned(1024))) char v_lds1[TILEB];

    const int N = p.N;                      // query rows per head
    const int Nk = SPLIT ? p.Nk : N;        // keys per head
    const int off = SPLIT ? p.q_off : 0;    // query i sits at key position i + off
    const int bhc = p.B * p.Hq;
    const int bkvc = p.B * p.Hkv;
    // Square forward: one unit per (batch, query head).  Split kernels: one unit per
    // (split, batch, K/V head), whose rows are those of the group's G query heads.
    const int units = SPLIT ? p.splits * bkvc : bhc;
    const int nqt = p.n_qtiles;
    const int bid = blockIdx.x;
    int u, qt;
    if (p.xcd_map) {
        int t;
        xcd_order(bid, units, nqt, u, t);
        qt = CAUSAL ? nqt - 1 - t : t;   // longest first
    } else {
        u = bid % units;
        qt = CAUSAL ? nqt - 1 - bid / units : bid / units;
    }
    const int split = SPLIT ? u / bkvc : 0;
    int b, hk, bh = 0;
    if constexpr (SPLIT) {
        const int bkv = u - split * bkvc;
        b = bkv / p.Hkv;
        hk = bkv - b * p.Hkv;
    } else {
        bh = u;
        b = bh / p.Hq;
        hk = (bh - b * p.Hq) / p.group;
    }
    // This workgroup's keys: [k_lo, k_hi), every key of the head unless split.
    const int k_lo = SPLIT ? split * p.chunk : 0;
    const int k_hi = SPLIT ? min(Nk, k_lo + p.chunk) : N;
    const char* Kh = (const char*)p.k + ((size_t)(b * p.Hkv + hk) * Nk + k_lo) * ROWB;
    const char* Vh = (const char*)p.v + ((size_t)(b * p.Hkv + hk) * Nk + k_lo) * ROWB;
    // Buffer ranges end at the head's last key: loads past it return zeros.
    const int range_bytes = k_hi > k_lo ? (Nk - k_lo) * ROWB : 0;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, range_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, range_bytes, 0x00020000);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // Optional clock stamps of this wave: the constant-rate real-time counter and the
    // shader-cycle counter, read at the start and at the end of the wave's work.
    unsigned long long real0 = 0, cyc0 = 0;
    if (!SPLIT && p.stamps) {
        real0 = __builtin_amdgcn_s_memrealtime();
        cyc0 = __builtin_amdgcn_s_memtime();
    }
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int q0 = qt * BM;
    const int qw0 = q0 + wave * 32;
    const int my_q = qw0 + l32;
    // Rows of this unit.  Square forward: row my_q of head bh.  Split kernels pack the
    // group: row r = g*N + i is query i of head hk*G + g, so one K/V tile serves every
    // query head that reads it (one query of each when decoding).  A row's result does
    // not depend on which rows share its tile.
    const int R = SPLIT ? p.group * N : N;           // rows of the unit
    const bool row_ok = my_q < R;
    int my_pos = my_q;                               // the row's query index i
    size_t qrow = (size_t)bh * N + my_q;             // flat [B][Hq][N] query row
    if constexpr (SPLIT) {
        const int g = my_q / N;
        my_pos = my_q - g * N;
        qrow = (size_t)(b * p.Hq + hk * p.group + g) * N + my_pos;
    }
    // Query indices the wave's (and the workgroup's) rows span: causal skipping uses the
    // largest, mask checks the smallest.
    auto pos_span = [&](int r_first, int r_last, int& pmin, int& pmax) {
        if (!SPLIT || r_first / N == r_last / N) {
            pmin = SPLIT ? r_first % N : r_first;
            pmax = SPLIT ? r_last % N : r_last;
        } else {
            pmin = 0;
            pmax = N - 1;
        }
    };
    int w_pmin, w_pmax, g_pmin, g_pmax;
    pos_span(qw0, SPLIT ? min(qw0 + 31, R - 1) : qw0 + 31, w_pmin, w_pmax);
    pos_span(q0, SPLIT ? min(q0 + BM - 1, R - 1) : q0 + BM - 1, g_pmin, g_pmax);
    (void)g_pmin;

    // Q as the B operand of S^T = K Q^T: dims 16kk + 8hi .. +7 of this lane's row.
    // A negative scale is folded into Q's sign so that c > 0 below; a zero scale
    // becomes the smallest normal float, which leaves every exp2 argument at 0.
    const float c = fmaxf(fabsf(p.scale_log2), FLT_MIN);
    const unsigned qflip = p.scale_log2 >= 0.f ? 0u : 0x80008000u;
    ex8 qf[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (row_ok) raw = *(const u32x4*)((const E*)p.q + qrow * D + 16 * kk + 8 * hi);
        raw ^= qflip;
        qf[kk] = __builtin_bit_cast(ex8, raw);
    }

    // Per-lane LDS byte offsets of the K operand: row 32t + l32, logical chunk 2kk + hi.
    const int kx = swz<D>(l32);
    int koff[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) koff[kk] = l32 * ROWB + 16 * ((2 * kk + hi) ^ kx);
    // V operand (transposed read): lane (group G, index 4j + s) addresses row
    // 32t + 16u + 8r + 4(G>>1) + j and dims 32dt + 16(G&1) + 4s .. +3.
    const int G = lane >> 4;
    const int jj = (lane >> 2) & 3;
    const int ss = lane & 3;
    int voff[2][DT];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int row = 8 * r + 4 * (G >> 1) + jj;
        const int w = swz<D>(row);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int chunk = 4 * dt + 2 * (G & 1) + (ss >> 1);
            voff[r][dt] = row * ROWB + 16 * (chunk ^ w) + 8 * (ss & 1);
        }
    }

    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m_ref = -INFINITY;   // exp reference, log2 units of the scaled score
    float l_run = 0.f;         // sum of P over this lane half's keys, against m_ref

    // Tiles of BN keys from k_lo; causal workgroups stop at their last row's diagonal.
    const int kv_end = CAUSAL ? min(k_hi, g_pmax + 1 + off) : k_hi;
    const int ntiles = kv_end > k_lo ? (kv_end - k_lo + BN - 1) / BN : 0;
    if constexpr (SPLIT) {
        if (ntiles == 0) {   // no row of this workgroup sees a key of this split: empty states
            if (row_ok) {
                float* Orow = (float*)p.o + ((size_t)split * bhc * N + qrow) * D;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *(float4*)(Orow + 32 * dt + 8 * g + 4 * hi) = make_float4(0.f, 0.f, 0.f, 0.f);
                if (hi == 0) p.lse[(size_t)split * bhc * N + qrow] = -INFINITY;
            }
            return;
        }
    }

    // Tile j of K (or V) into buffer BUF, straight from HBM into LDS.
    auto issue_k = [&](int j, auto bufsel) {
        char* dst = decltype(bufsel)::value == 0 ? k_lds0 : k_lds1;
#pragma unroll
        for (int i = 0; i < LOADS / NW; ++i) {
            const int ii = wave + i * NW;                 // which 1 KiB slice of the tile
            const int off = ii * 1024 + 16 * lane;        // this lane's physical bytes
            const int row = off / ROWB;
            const int chunk = ((off % ROWB) >> 4) ^ swz<D>(row);
            const unsigned src = (unsigned)((j * BN + row) * ROWB + 16 * chunk);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (FA_LDS void*)(dst + ii * 1024), 16, src, 0, 0, 0);
        }
    };
    auto issue_v = [&](int j, auto bufsel) {
        char* dst = decltype(bufsel)::value == 0 ? v_lds0 : v_lds1;
#pragma unroll
        for (int i = 0; i < LOADS / NW; ++i) {
            const int ii = wave + i * NW;
            const int off = ii * 1024 + 16 * lane;
            const int row = off / ROWB;
            const int chunk = ((off % ROWB) >> 4) ^ swz<D>(row);
            const unsigned src = (unsigned)((j * BN + row) * ROWB + 16 * chunk);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (FA_LDS void*)(dst + ii * 1024), 16, src, 0, 0, 0);
        }
    };

    // S^T of one key tile from the K buffer BUF.
    auto s_tile = [&](f32x16 (&s)[ST], auto bufsel) {
        const char* kb = decltype(bufsel)::value == 0 ? k_lds0 : k_lds1;
#pragma unroll
        for (int t = 0; t < ST; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[t][r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) {
                const ex8 a = *(const FA_LDS ex8*)(kb + 32 * t * ROWB + koff[kk]);
                s[t] = Elem<E>::mfma(a, qf[kk], s[t]);
            }
        }
    };

    // -inf for keys this lane's row may not see (only ever needed on a wave's last tile).
    auto mask_tile = [&](f32x16 (&s)[ST], int j) {
        const int lim = (CAUSAL ? min(my_pos + off, Nk - 1) : Nk - 1) - (k_lo + j * BN + 4 * hi);   // relative last key
#pragma unroll
        for (int t = 0; t < ST; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (32 * t + 8 * (r >> 2) + (r & 3) > lim) s[t][r] = -INFINITY;
    };

    // Online-softmax update for one tile of scores: returns the rescale factor for O
    // (1 where the reference did not move) and whether any row of the wave moved.
    auto softmax = [&](f32x16 (&s)[ST], ex8 (&pb)[ST][2], float& alpha) -> bool {
        float mx0 = s[0][0], mx1 = s[0][1];
#pragma unroll
        for (int t = 0; t < ST; ++t)
#pragma unroll
            for (int r = (t == 0 ? 2 : 0); r < 16; r += 2) {
                mx0 = fmaxf(mx0, s[t][r]);
                mx1 = fmaxf(mx1, s[t][r + 1]);
            }
        const float mx = lane_half_max(fmaxf(mx0, mx1)) * c;
        // lazy rescale: move the reference only when the max has grown past the slack
        const bool grow = mx > m_ref + kRescaleSlack;
        const float m_new = grow ? mx : m_ref;
        alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
        m_ref = m_new;
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;   // nothing finite yet: P = 0
        // Row sums in fp32 vector adds, four chains: the pair dot product (v_dot2) would
        // wait for the matrix products in flight on the SIMD.
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < ST; ++t)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][8 * u + e], c, -m_use));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][8 * u + e + 1], c, -m_use));
                    pb[t][u][e] = (E)p0;
                    pb[t][u][e + 1] = (E)p1;
                    ls[e >> 1] += p0 + p1;
                }
        l_run = l_run * alpha + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
        return __builtin_amdgcn_ballot_w64(grow) != 0;
    };

    auto rescale_o = [&](float alpha) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    };

    // O^T += V_tile^T P^T from the V buffer BUF.
    auto pv = [&](const ex8 (&pb)[ST][2], auto bufsel) {
        const char* vb = decltype(bufsel)::value == 0 ? v_lds0 : v_lds1;
#pragma unroll
        for (int t = 0; t < ST; ++t)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const char* vrow = vb + (32 * t + 16 * u) * ROWB;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(vrow + voff[0][dt]));
                    const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(vrow + voff[1][dt]));
                    const i16x8 both = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
                    o[dt] = Elem<E>::mfma(__builtin_bit_cast(ex8, both), pb[t][u], o[dt]);
                }
    };

    // Software pipeline, per wave: while tile j's softmax runs on the VALU, tile j+1's
    // scores run on the MFMA unit; then tile j's PV product.  Iteration j reads K_{j+1}
    // and V_j and loads K_{j+2} and V_{j+1}, so K runs one tile ahead of V.  A wave's only
    // masked tile is its last one (the tile holding its diagonal, or the N tail), so the
    // steady-state iteration carries no mask code.
    // The wave's last tile: the one holding its last row's diagonal (causal), else the
    // last; -1 when the wave has no row below N or no visible key in this range.
    int my_last = ntiles - 1;
    if (CAUSAL) {
        const int last_key = w_pmax + off;
        my_last = last_key < k_lo ? -1 : min(ntiles - 1, (last_key - k_lo) / BN);
    }
    if (qw0 >= R) my_last = -1;
    // Scores of tile j live in sa for even j and in sb for odd j: no copies between tiles.
    f32x16 sa[ST], sb[ST];

    auto iter = [&](int j, auto par, f32x16 (&s_cur)[ST], f32x16 (&s_nxt)[ST]) {
        constexpr int P = decltype(par)::value;     // j & 1: V_j in V buffer P, K_{j+1} in K buffer 1-P
        tile_barrier();                            // K_{j+1} and V_j landed; K_j and V_{j-1} are free
        if (j + 2 < ntiles) issue_k(j + 2, Int<P>{});
        if (j + 1 < ntiles) issue_v(j + 1, Int<1 - P>{});
        if (j > my_last) return;                   // this wave's rows are done
        ex8 pb[ST][2];
        float alpha;
        bool any;
        if (j < my_last) {
            s_tile(s_nxt, Int<1 - P>{});
            if constexpr (SPLIT && CAUSAL) {   // the diagonal may straddle this tile and the next
                if (k_lo + j * BN + BN - 1 > w_pmin + off) mask_tile(s_cur, j);
            }
            any = softmax(s_cur, pb, alpha);
        } else {
            if ((CAUSAL && k_lo + j * BN + BN - 1 > w_pmin + off) || (k_lo + j * BN + BN > Nk)) mask_tile(s_cur, j);
            any = softmax(s_cur, pb, alpha);
        }
        if (any) rescale_o(alpha);
        pv(pb, Int<P>{});
    };

    issue_k(0, Int<0>{});
    issue_v(0, Int<0>{});
    if (ntiles > 1) issue_k(1, Int<1>{});
    tile_barrier();
    s_tile(sa, Int<0>{});                          // every wave sees key 0
    for (int j = 0; j < ntiles; j += 2) {
        iter(j, Int<0>{}, sa, sb);
        if (j + 1 < ntiles) iter(j + 1, Int<1>{}, sb, sa);
    }

    // epilogue: O = u / l, LSE = m + ln l
    const float l_tot = lane_half_sum(l_run);
    if constexpr (SPLIT) {
        if (row_ok) {   // float partial state; l = 0 marks a row with no visible key here
            const bool empty = !(l_tot > 0.f);
            const float inv = empty ? 0.f : 1.f / l_tot;
            float* Orow = (float*)p.o + ((size_t)split * bhc * N + qrow) * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *(float4*)(Orow + 32 * dt + 8 * g + 4 * hi) =
                        make_float4(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, o[dt][4 * g + 2] * inv,
                                    o[dt][4 * g + 3] * inv);
            if (hi == 0)
                p.lse[(size_t)split * bhc * N + qrow] = empty ? -INFINITY : (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
        }
        return;
    }
    if (my_q < N) {
        const float inv = 1.f / l_tot;
        E* Orow = (E*)p.o + (size_t)bh * N * D + (size_t)my_q * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                ex4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (E)(o[dt][4 * g + e] * inv);
                *(ex4*)(Orow + 32 * dt + 8 * g + 4 * hi) = w;
            }
        if (hi == 0) p.lse[(size_t)bh * N + my_q] = (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    if (p.stamps && lane == 0) {
        const unsigned long long cyc1 = __builtin_amdgcn_s_memtime();
        const unsigned long long real1 = __builtin_amdgcn_s_memrealtime();
        typedef __attribute__((ext_vector_type(4))) unsigned long long u64x4;
        *(u64x4*)(p.stamps + ((size_t)bid * NW + wave) * 4) = u64x4{real0, real1, cyc0, cyc1};
    }
}

// Explicit instantiations: both the host and the device pass must see every
// kernel the dispatch tables name.
#define FA16_INSTANTIATE(E, D, BM, BN, SPLIT)                                                 \
    template __global__ void fwd16_kernel<E, D, BM, BN, false, SPLIT>(const FwdParams);   \
    template __global__ void fwd16_kernel<E, D, BM, BN, true, SPLIT>(const FwdParams);
#define FA16_INSTANTIATE_TYPE(E)                \
    FA16_INSTANTIATE(E, 128, 128, 64, false)    \
    FA16_INSTANTIATE(E, 128, 128, 32, false)    \
    FA16_INSTANTIATE(E, 64, 128, 64, false)     \
    FA16_INSTANTIATE(E, 64, 128, 32, false)     \
    FA16_INSTANTIATE(E, 128, 128, 64, true)     \
    FA16_INSTANTIATE(E, 64, 128, 64, true)
FA16_INSTANTIATE_TYPE(__bf16)
FA16_INSTANTIATE_TYPE(_Float16)

namespace {

template <typename E, int D, int BM, int BN, bool CAUSAL, bool SPLIT>
hipError_t launch16(const FwdParams& p, hipStream_t stream)
{
    const long long units = SPLIT ? (long long)p.splits * p.B * p.Hkv : (long long)p.B * p.Hq;
    const long long grid = units * p.n_qtiles;
    FwdParams args = p;
    args.xcd_map = (units % 8 == 0) ? 1 : 0;   // needs whole heads per XCD
    void* kargs[] = {&args};
    return hipLaunchKernel((const void*)&fwd16_kernel<E, D, BM, BN, CAUSAL, SPLIT>, dim3((unsigned)grid),
                           dim3(BM * 2), kargs, 0, stream);
}

}  // namespace

// The dispatch tables are host data: they are not emitted in the device pass.
#if !defined(__HIP_DEVICE_COMPILE__)
#define FA16_ENTRY(E, DT, D, BM, BN, SPLIT)                                   \
    {DT, D, BM, BN, 0, &launch16<E, D, BM, BN, false, SPLIT>},               \
    {DT, D, BM, BN, 1, &launch16<E, D, BM, BN, true, SPLIT>}

// The first shape listed for each head dimension is the default.
#define FA16_TABLE(E, DT)                          \
    FA16_ENTRY(E, DT, 128, 128, 64, false),        \
    FA16_ENTRY(E, DT, 128, 128, 32, false),        \
    FA16_ENTRY(E, DT, 64, 128, 64, false),         \
    FA16_ENTRY(E, DT, 64, 128, 32, false)
#define FA16_SPLIT_TABLE(E, DT)                    \
    FA16_ENTRY(E, DT, 128, 128, 64, true),         \
    FA16_ENTRY(E, DT, 64, 128, 64, true)

const KernelEntry kBf16Kernels[] = {FA16_TABLE(__bf16, 1)};
const int kNumBf16Kernels = sizeof(kBf16Kernels) / sizeof(kBf16Kernels[0]);
const KernelEntry kF16Kernels[] = {FA16_TABLE(_Float16, 2)};
const int kNumF16Kernels = sizeof(kF16Kernels) / sizeof(kF16Kernels[0]);
const KernelEntry kBf16SplitKernels[] = {FA16_SPLIT_TABLE(__bf16, 1)};
const int kNumBf16SplitKernels = sizeof(kBf16SplitKernels) / sizeof(kBf16SplitKernels[0]);
const KernelEntry kF16SplitKernels[] = {FA16_SPLIT_TABLE(_Float16, 2)};
const int kNumF16SplitKernels = sizeof(kF16SplitKernels) / sizeof(kF16SplitKernels[0]);

#endif

}  // namespace fa
