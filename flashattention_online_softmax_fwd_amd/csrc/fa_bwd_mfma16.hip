// fa_bwd_mfma16.hip -- backward pass of exact attention for gfx950 (CDNA4, MI355X),
// 16-bit inputs (bf16 or fp16), fp32 accumulation.
//
// The score matrix is not stored by the forward; it is recomputed here from Q, K and
// the forward's LSE (the paweldubiel.com FlashAttention note, "Mechanism and
// details": training recomputes quantities in the backward pass instead of storing
// them; the spicyshark.co lesson, "Further reading").  With c = scale * log2(e):
//     P  = exp2(c * q.k - LSE * log2(e))        (exactly softmax(scale * q K^T), masked keys 0)
//     D  = rowsum(dO * O)
//     dP = dO v^T,  dS = P * (dP - D)
//     dQ = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO
// the exact gradient of O = softmax(scale Q K^T) V.  Two kernels, in stream order:
//   dq      one workgroup per 128 query rows (4 waves x 32): D of each row from its O
//           and dO (written to the caller's delta buffer), then a loop over key tiles
//           as the forward's: S^T = K Q^T and dP^T = V dO^T, dS^T, then
//           dQ^T += K^T dS^T (K^T from transposed LDS reads);
//   dkdv    one workgroup per 128 keys (4 waves x 32), looping over 32-query tiles
//           of every query head that reads this K/V head: S = Q K^T and dP = dO V^T,
//           so one key per lane and the rounded P and dS are directly the B operands
//           of dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T from transposed reads).
//           When the grid is small, each key tile's query tiles are shared out over S
//           workgroups that write fp32 partial sums; a last kernel adds the S partials
//           of every element in split order and rounds them.
// Every output element is accumulated by one wave in a fixed order: no atomics,
// results reproducible bit for bit.  LDS tiles use the forward's layout (16-byte
// chunks XOR-swizzled per row, filled by buffer_load ... lds).
#include "fa_kernels.h"
#include "fa_mfma16_common.h"

#include <float.h>
#include <stdint.h>

#include <mutex>

namespace fa {
namespace bwd {
constexpr float kLog2e = 1.4426950408889634f;
typedef __attribute__((ext_vector_type(4))) float f32x4;
}

// dQ: per query tile of 128 rows, over the key tiles the rows see.
template <typename E, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_kernel(const BwdParams p)
{
    typedef typename Elem<E>::x8 ex8;
    typedef typename Elem<E>::x4 ex4;
    typedef typename Elem<E>::x2 ex2;
    constexpr int BM = 128, BN = 64, NW = 4;
    constexpr int ROWB = D * 2;
    constexpr int TILEB = BN * ROWB;
    constexpr int LOADS = TILEB / 1024;
    constexpr int DK = D / 16;
    constexpr int ST = BN / 32;
    constexpr int DT = D / 32;
    static_assert(LOADS % NW == 0, "tile loads must split evenly over the waves");

    __shared__ __attribute__((aligned(1024))) char k_lds0[TILEB];
    __shared__ __attribute__((aligned(1024))) char k_lds1[TILEB];
    __shared__ __attribute__((aligned(1024))) char v_lds0[TILEB];
    __shared__ __attribute__((aligned(1024))) char v_lds1[TILEB];

    const int N = p.N;
    const int bhc = p.B * p.Hq;
    const int nqt = (N + BM - 1) / BM;
    const int bid = blockIdx.x;
    int bh, qt;
    if (p.xcd_map) {
        int t;
        xcd_order(bid, bhc, nqt, bh, t);
        qt = CAUSAL ? nqt - 1 - t : t;   // longest first
    } else {
        bh = bid % bhc;
        qt = CAUSAL ? nqt - 1 - bid / bhc : bid / bhc;
    }
    const int b = bh / p.Hq;
    const int hk = (bh - b * p.Hq) / p.group;
    const char* Kh = (const char*)p.k + (size_t)(b * p.Hkv + hk) * N * ROWB;
    const char* Vh = (const char*)p.v + (size_t)(b * p.Hkv + hk) * N * ROWB;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, N * ROWB, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, N * ROWB, 0x00020000);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int q0 = qt * BM;
    const int qw0 = q0 + wave * 32;
    const int my_q = qw0 + l32;
    const bool row_ok = my_q < N;
    const size_t qrow = (size_t)bh * N + my_q;

    // This lane's rows of Q and dO as B operands (dims 16kk + 8hi .. +7), its LSE in
    // log2 units and its D.
    ex8 qf[DK], gf[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
        u32x4 rq = {0u, 0u, 0u, 0u}, rg = {0u, 0u, 0u, 0u};
        if (row_ok) {
            rq = *(const u32x4*)((const E*)p.q + qrow * D + 16 * kk + 8 * hi);
            rg = *(const u32x4*)((const E*)p.dout + qrow * D + 16 * kk + 8 * hi);
        }
        qf[kk] = __builtin_bit_cast(ex8, rq);
        gf[kk] = __builtin_bit_cast(ex8, rg);
    }
    const float c = p.scale * bwd::kLog2e;
    const float lse2 = row_ok ? p.lse[qrow] * bwd::kLog2e : 0.f;
    // D = rowsum(dO * O) of this lane's row: each lane half takes its 64 (or 32) dims,
    // then one swap.  Written for the dK/dV kernel, which runs next on the stream.
    float dpart = 0.f;
    if (row_ok) {
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) {
            const ex8 ov = __builtin_bit_cast(ex8, *(const u32x4*)((const E*)p.o + qrow * D + 16 * kk + 8 * hi));
#pragma unroll
            for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf((float)ov[e], (float)gf[kk][e], dpart);
        }
    }
    const float dlt = lane_half_sum(dpart);
    if (row_ok && hi == 0) p.delta[qrow] = dlt;

    const int kx = swz<D>(l32);
    int koff[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) koff[kk] = l32 * ROWB + 16 * ((2 * kk + hi) ^ kx);
    const int G = lane >> 4;
    const int jj = (lane >> 2) & 3;
    const int ss = lane & 3;
    int toff[2][DT];   // transposed reads: 4 rows x 16 columns across each 16-lane group
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int row = 8 * r + 4 * (G >> 1) + jj;
        const int w = swz<D>(row);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int chunk = 4 * dt + 2 * (G & 1) + (ss >> 1);
            toff[r][dt] = row * ROWB + 16 * (chunk ^ w) + 8 * (ss & 1);
        }
    }

    f32x16 dq[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kv_end + BN - 1) / BN;
    int my_last = CAUSAL ? min(ntiles - 1, (qw0 + 31) / BN) : ntiles - 1;
    if (qw0 >= N) my_last = -1;

    auto issue = [&](const __amdgpu_buffer_rsrc_t& rs, char* dst, int j) {
#pragma unroll
        for (int i = 0; i < LOADS / NW; ++i) {
            const int ii = wave + i * NW;
            const int off = ii * 1024 + 16 * lane;
            const int row = off / ROWB;
            const int chunk = ((off % ROWB) >> 4) ^ swz<D>(row);
            const unsigned src = (unsigned)((j * BN + row) * ROWB + 16 * chunk);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)(dst + ii * 1024), 16, src, 0, 0, 0);
        }
    };

    auto iter = [&](int j, auto par) {
        constexpr int P = decltype(par)::value;
        const char* kb = P == 0 ? k_lds0 : k_lds1;
        const char* vb = P == 0 ? v_lds0 : v_lds1;
        tile_barrier();                                      // K_j, V_j landed; buffers 1-P free
        if (j + 1 < ntiles) {
            issue(krs, P == 0 ? k_lds1 : k_lds0, j + 1);
            issue(vrs, P == 0 ? v_lds1 : v_lds0, j + 1);
        }
        if (j > my_last) return;
        f32x16 s[ST], dp[ST];
#pragma unroll
        for (int t = 0; t < ST; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[t][r] = 0.f;
                dp[t][r] = 0.f;
            }
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) {
                const ex8 a = *(const FA_LDS ex8*)(kb + 32 * t * ROWB + koff[kk]);
                const ex8 bv = *(const FA_LDS ex8*)(vb + 32 * t * ROWB + koff[kk]);
                s[t] = Elem<E>::mfma(a, qf[kk], s[t]);
                dp[t] = Elem<E>::mfma(bv, gf[kk], dp[t]);
            }
        }
        // dS^T = P^T (dP^T - D), P^T = exp2(c s - lse2); keys past the row's diagonal or N get 0
        const bool masked = (CAUSAL && j * BN + BN - 1 > qw0) || (j * BN + BN > N);
        const int lim = (CAUSAL ? min(my_q, N - 1) : N - 1) - (j * BN + 4 * hi);
        ex8 dsb[ST][2];
#pragma unroll
        for (int t = 0; t < ST; ++t)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    float v2[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int r = 8 * u + e + h;
                        float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, -lse2));
                        if (masked && 32 * t + 8 * (r >> 2) + (r & 3) > lim) pr = 0.f;
                        v2[h] = pr * (dp[t][r] - dlt);
                    }
                    ex2 pair;
                    pair[0] = (E)v2[0];
                    pair[1] = (E)v2[1];
                    dsb[t][u][e] = pair[0];
                    dsb[t][u][e + 1] = pair[1];
                }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int t = 0; t < ST; ++t)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const char* krow = kb + (32 * t + 16 * u) * ROWB;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(krow + toff[0][dt]));
                    const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(krow + toff[1][dt]));
                    const i16x8 both = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
                    dq[dt] = Elem<E>::mfma(__builtin_bit_cast(ex8, both), dsb[t][u], dq[dt]);
                }
    };

    issue(krs, k_lds0, 0);
    issue(vrs, v_lds0, 0);
    for (int j = 0; j < ntiles; j += 2) {
        iter(j, Int<0>{});
        if (j + 1 < ntiles) iter(j + 1, Int<1>{});
    }

    if (row_ok) {
        E* dst = (E*)p.dq + qrow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                ex4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (E)(dq[dt][4 * g + e] * p.scale);
                *(ex4*)(dst + 32 * dt + 8 * g + 4 * hi) = w;
            }
    }
}

// dK and dV: per tile of 128 keys of one K/V head, over the 32-query tiles of every
// query head that reads it.
template <typename E, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_kernel(const BwdParams p)
{
    typedef typename Elem<E>::x8 ex8;
    typedef typename Elem<E>::x4 ex4;
    typedef typename Elem<E>::x2 ex2;
    constexpr int BK = 128, BQ = 32, NW = 4;
    constexpr int ROWB = D * 2;
    constexpr int QTILEB = BQ * ROWB;
    constexpr int QLOADS = QTILEB / 1024;
    constexpr int VTILEB = BK * ROWB;
    constexpr int VLOADS = VTILEB / 1024;
    constexpr int DK = D / 16;
    constexpr int DT = D / 32;
    static_assert(QLOADS % NW == 0 && VLOADS % NW == 0, "tile loads must split evenly over the waves");

    __shared__ __attribute__((aligned(1024))) char v_lds[VTILEB];
    __shared__ __attribute__((aligned(1024))) char q_lds0[QTILEB];
    __shared__ __attribute__((aligned(1024))) char q_lds1[QTILEB];
    __shared__ __attribute__((aligned(1024))) char g_lds0[QTILEB];
    __shared__ __attribute__((aligned(1024))) char g_lds1[QTILEB];
    __shared__ __attribute__((aligned(256))) float ls_lds0[64];   // LSE of the tile's queries (first 32 used)
    __shared__ __attribute__((aligned(256))) float ls_lds1[64];
    __shared__ __attribute__((aligned(256))) float dl_lds0[64];   // their D
    __shared__ __attribute__((aligned(256))) float dl_lds1[64];

    const int N = p.N;
    const int Gq = p.group;
    const int bkvc = p.B * p.Hkv;
    const int nkt = (N + BK - 1) / BK;
    const int S = p.splits;
    const int bid = blockIdx.x;
    int bkv, kts;   // kts = kt * S + split: the splits of one key tile are adjacent
    if (p.xcd_map) {
        xcd_order(bid, bkvc, nkt * S, bkv, kts);   // causal: early key tiles see the most queries
    } else {
        bkv = bid % bkvc;
        kts = bid / bkvc;
    }
    const int kt = kts / S;
    const int split = kts - kt * S;
    const int b = bkv / p.Hkv;
    const int hk = bkv - b * p.Hkv;
    const int k0 = kt * BK;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int kw0 = k0 + wave * 32;
    const int my_k = kw0 + l32;
    const size_t krow = (size_t)bkv * N + my_k;

    // This lane's key row of K as the B operand of S = Q K^T.
    ex8 kf[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (my_k < N) raw = *(const u32x4*)((const E*)p.k + krow * D + 16 * kk + 8 * hi);
        kf[kk] = __builtin_bit_cast(ex8, raw);
    }
    const float c = p.scale * bwd::kLog2e;

    const int kx = swz<D>(l32);
    int koff[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) koff[kk] = l32 * ROWB + 16 * ((2 * kk + hi) ^ kx);
    const int G = lane >> 4;
    const int jj = (lane >> 2) & 3;
    const int ss = lane & 3;
    int toff[2][DT];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int row = 8 * r + 4 * (G >> 1) + jj;
        const int w = swz<D>(row);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int chunk = 4 * dt + 2 * (G & 1) + (ss >> 1);
            toff[r][dt] = row * ROWB + 16 * (chunk ^ w) + 8 * (ss & 1);
        }
    }

    f32x16 dk[DT], dv[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk[dt][r] = 0.f;
            dv[dt][r] = 0.f;
        }

    // Query tiles: for each of the G query heads of this K/V head, the 32-query tiles
    // from the first that can see one of this workgroup's keys.
    const int nq = (N + BQ - 1) / BQ;
    const int qi0 = CAUSAL ? k0 / BQ : 0;
    const int per_head = nq - qi0;
    // With S splits, split s takes a contiguous share of the G * per_head tiles.
    const int all_tiles = Gq * per_head;
    const int share = (all_tiles + S - 1) / S;
    const int t_lo = min(all_tiles, split * share);
    const int t_hi = min(all_tiles, t_lo + share);

    // V rows of this key tile into LDS once.
    {
        const char* Vh = (const char*)p.v + ((size_t)bkv * N + k0) * ROWB;
        const __amdgpu_buffer_rsrc_t vrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, (N - k0) * ROWB, 0x00020000);
#pragma unroll
        for (int i = 0; i < VLOADS / NW; ++i) {
            const int ii = wave + i * NW;
            const int off = ii * 1024 + 16 * lane;
            const int row = off / ROWB;
            const int chunk = ((off % ROWB) >> 4) ^ swz<D>(row);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (FA_LDS void*)(v_lds + ii * 1024), 16,
                                                     (unsigned)(row * ROWB + 16 * chunk), 0, 0, 0);
        }
    }

    // Tile t: Q and dO rows i0 .. i0+31 of query head hk*G + g, their LSE and D.
    auto issue = [&](int t, char* qd, char* gd, float* ld, float* dd) {
        const int g = t / per_head;
        const int i0 = (qi0 + t % per_head) * BQ;
        const size_t hrow = (size_t)(b * p.Hq + hk * Gq + g) * N;
        const __amdgpu_buffer_rsrc_t qrs =
            __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.q + hrow * ROWB), (short)0, N * ROWB, 0x00020000);
        const __amdgpu_buffer_rsrc_t grs =
            __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.dout + hrow * ROWB), (short)0, N * ROWB, 0x00020000);
#pragma unroll
        for (int i = 0; i < QLOADS / NW; ++i) {
            const int ii = wave + i * NW;
            const int off = ii * 1024 + 16 * lane;
            const int row = off / ROWB;
            const int chunk = ((off % ROWB) >> 4) ^ swz<D>(row);
            const unsigned src = (unsigned)((i0 + row) * ROWB + 16 * chunk);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (FA_LDS void*)(qd + ii * 1024), 16, src, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(grs, (FA_LDS void*)(gd + ii * 1024), 16, src, 0, 0, 0);
        }
        if (wave == 0) {   // 64 lanes x 4 bytes: queries i0 .. i0+63 (the tile uses the first 32)
            const __amdgpu_buffer_rsrc_t lrs =
                __builtin_amdgcn_make_buffer_rsrc((void*)(p.lse + hrow), (short)0, N * 4, 0x00020000);
            const __amdgpu_buffer_rsrc_t drs =
                __builtin_amdgcn_make_buffer_rsrc((void*)(p.delta + hrow), (short)0, N * 4, 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (FA_LDS void*)ld, 4, (unsigned)((i0 + lane) * 4), 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (FA_LDS void*)dd, 4, (unsigned)((i0 + lane) * 4), 0, 0, 0);
        }
    };

    auto iter = [&](int t, auto par) {
        constexpr int P = decltype(par)::value;
        const char* qb = P == 0 ? q_lds0 : q_lds1;
        const char* gb = P == 0 ? g_lds0 : g_lds1;
        const float* lb = P == 0 ? ls_lds0 : ls_lds1;
        const float* db = P == 0 ? dl_lds0 : dl_lds1;
        tile_barrier();                                   // tile t (and V) landed; buffers 1-P free
        if (t + 1 < t_hi) {
            if constexpr (P == 0) issue(t + 1, q_lds1, g_lds1, ls_lds1, dl_lds1);
            else issue(t + 1, q_lds0, g_lds0, ls_lds0, dl_lds0);
        }
        const int i0 = (qi0 + t % per_head) * BQ;
        if (CAUSAL && i0 + BQ - 1 < kw0) return;           // every query of the tile precedes this wave's keys
        if (kw0 >= N) return;
        // S = Q K^T and dP = dO V^T: lane l32 holds key my_k, register r query i0 + 8(r/4) + 4hi + r%4
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = 0.f;
            dp[r] = 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) {
            const ex8 a = *(const FA_LDS ex8*)(qb + koff[kk]);
            const ex8 ag = *(const FA_LDS ex8*)(gb + koff[kk]);
            const ex8 vw = *(const FA_LDS ex8*)(v_lds + wave * 32 * ROWB + koff[kk]);
            s = Elem<E>::mfma(a, kf[kk], s);
            dp = Elem<E>::mfma(ag, vw, dp);
        }
        // P = exp2(c s - LSE log2 e), 0 for masked queries; dS = P (dP - D)
        const bool masked = (CAUSAL && i0 < kw0 + 31) || (i0 + BQ > N);
        ex8 pb[2], dsb[2];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const bwd::f32x4 lv = *(const FA_LDS bwd::f32x4*)(lb + 8 * q4 + 4 * hi);
            const bwd::f32x4 dv4 = *(const FA_LDS bwd::f32x4*)(db + 8 * q4 + 4 * hi);
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                float pv[2], sv[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 4 * q4 + e + h;
                    const int qi = i0 + 8 * q4 + 4 * hi + e + h;
                    float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lv[e + h] * bwd::kLog2e));
                    if (masked && (qi >= N || (CAUSAL && qi < my_k))) pr = 0.f;
                    pv[h] = pr;
                    sv[h] = pr * (dp[r] - dv4[e + h]);
                }
                const int u = q4 >> 1;
                const int slot = 4 * (q4 & 1) + e;
                ex2 pp, dd2;
                pp[0] = (E)pv[0];
                pp[1] = (E)pv[1];
                dd2[0] = (E)sv[0];
                dd2[1] = (E)sv[1];
                pb[u][slot] = pp[0];
                pb[u][slot + 1] = pp[1];
                dsb[u][slot] = dd2[0];
                dsb[u][slot + 1] = dd2[1];
            }
        }
        // dV^T += dO^T P and dK^T += Q^T dS, the transposed operands from LDS
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const char* grow = gb + 16 * u * ROWB;
                const char* qrow = qb + 16 * u * ROWB;
                const i16x4 glo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(grow + toff[0][dt]));
                const i16x4 gup = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(grow + toff[1][dt]));
                const i16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(qrow + toff[0][dt]));
                const i16x4 qup = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(qrow + toff[1][dt]));
                const i16x8 gboth = {glo[0], glo[1], glo[2], glo[3], gup[0], gup[1], gup[2], gup[3]};
                const i16x8 qboth = {qlo[0], qlo[1], qlo[2], qlo[3], qup[0], qup[1], qup[2], qup[3]};
                dv[dt] = Elem<E>::mfma(__builtin_bit_cast(ex8, gboth), pb[u], dv[dt]);
                dk[dt] = Elem<E>::mfma(__builtin_bit_cast(ex8, qboth), dsb[u], dk[dt]);
            }
    };

    if (t_lo < t_hi) issue(t_lo, q_lds0, g_lds0, ls_lds0, dl_lds0);
    for (int t = t_lo; t < t_hi; t += 2) {
        iter(t, Int<0>{});
        if (t + 1 < t_hi) iter(t + 1, Int<1>{});
    }
    tile_barrier();   // the V load above, when no tile was processed

    if (S > 1) {   // fp32 partial sums, added up in split order by the reduce kernel
        if (my_k < N) {
            const size_t plane = (size_t)S * bkvc * N * D;
            float* pk = p.dkv_part + ((size_t)split * bkvc * N + krow) * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float4 wk, wv;
                    wk.x = dk[dt][4 * g] * p.scale;
                    wk.y = dk[dt][4 * g + 1] * p.scale;
                    wk.z = dk[dt][4 * g + 2] * p.scale;
                    wk.w = dk[dt][4 * g + 3] * p.scale;
                    wv.x = dv[dt][4 * g];
                    wv.y = dv[dt][4 * g + 1];
                    wv.z = dv[dt][4 * g + 2];
                    wv.w = dv[dt][4 * g + 3];
                    *(float4*)(pk + 32 * dt + 8 * g + 4 * hi) = wk;
                    *(float4*)(pk + plane + 32 * dt + 8 * g + 4 * hi) = wv;
                }
        }
        return;
    }
    if (my_k < N) {
        E* dkr = (E*)p.dk + krow * D;
        E* dvr = (E*)p.dv + krow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                ex4 wk, wv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wk[e] = (E)(dk[dt][4 * g + e] * p.scale);
                    wv[e] = (E)dv[dt][4 * g + e];
                }
                *(ex4*)(dkr + 32 * dt + 8 * g + 4 * hi) = wk;
                *(ex4*)(dvr + 32 * dt + 8 * g + 4 * hi) = wv;
            }
    }
}

// dK and dV from S fp32 partials: out = sum over s of part[s], in split order.
// part is [2][S][rows][D] (dK planes, then dV planes); one thread per 8 elements.
template <typename E, int D>
__global__ void __launch_bounds__(256) bwd_reduce_kernel(const BwdParams p)
{
    typedef typename Elem<E>::x8 ex8;
    const long long rows = (long long)p.B * p.Hkv * p.N;
    const long long per_plane = rows * D / 8;                 // 8-element groups in dK (or dV)
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= 2 * per_plane) return;
    const int which = i >= per_plane ? 1 : 0;                 // 0: dK, 1: dV
    const long long e0 = (i - which * per_plane) * 8;
    const size_t split_stride = (size_t)rows * D;
    const float* src = p.dkv_part + (size_t)which * p.splits * split_stride + e0;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int sp = 0; sp < p.splits; ++sp) {
        const float4 a = *(const float4*)(src + sp * split_stride);
        const float4 b = *(const float4*)(src + sp * split_stride + 4);
        acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
        acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    ex8 w;
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = (E)acc[e];
    *(ex8*)((E*)(which ? p.dv : p.dk) + e0) = w;
}

#define FA_BWD_INSTANTIATE(E, D)                                                   \
    template __global__ void bwd_dq_kernel<E, D, false>(const BwdParams);         \
    template __global__ void bwd_dq_kernel<E, D, true>(const BwdParams);          \
    template __global__ void bwd_dkdv_kernel<E, D, false>(const BwdParams);       \
    template __global__ void bwd_dkdv_kernel<E, D, true>(const BwdParams);       \
    template __global__ void bwd_reduce_kernel<E, D>(const BwdParams);
FA_BWD_INSTANTIATE(__bf16, 128)
FA_BWD_INSTANTIATE(__bf16, 64)
FA_BWD_INSTANTIATE(_Float16, 128)
FA_BWD_INSTANTIATE(_Float16, 64)

// The workspace of the allocation-free split backward (fa_bwd_split_noalloc): room for
// the fp32 dK/dV partials [2][splits][B][Hkv][N][d] of calls up to kBwdScratchBytes.
// Each GPU holds its own copy from the moment the library's code is loaded on it
// until the process ends.  Every dK/dV workgroup writes its whole share of it, so
// nothing has to be cleared between calls; calls that overlap on one GPU race.
static __device__ __align__(256) float scratch[kBwdScratchBytes / sizeof(float)];

// The lookup below is compiled in both passes: the device pass must see that host code
// takes the array's address, or it drops the array as unused and the runtime then has
// no device symbol behind the name.
namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
float* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

}  // namespace

hipError_t bwd_scratch(hipStream_t stream, float** ptr)
{
    int dev = 0;
    hipError_t err = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    // Once per device, with that device current: in host code the array's name is only a
    // stand-in, so its device address is looked up and kept.
    std::call_once(g_scratch_once[dev], [dev]() {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        if (e == hipSuccess) e = hipGetSymbolAddress((void**)&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e == hipSuccess && !g_scratch_ptr[dev]) e = hipErrorInvalidSymbol;
        g_scratch_err[dev] = e;
    });
    *ptr = g_scratch_ptr[dev];
    return g_scratch_err[dev];
}

#if !defined(__HIP_DEVICE_COMPILE__)
namespace {
template <typename E, int D>
hipError_t launch_bwd_t(const BwdParams& p0, int causal, hipStream_t stream)
{
    BwdParams p = p0;
    void* kargs[] = {&p};
    const long long nqt = (p.N + 127) / 128;
    p.xcd_map = ((long long)p.B * p.Hq) % 8 == 0 ? 1 : 0;
    hipError_t err = hipLaunchKernel(causal ? (const void*)&bwd_dq_kernel<E, D, true> : (const void*)&bwd_dq_kernel<E, D, false>,
                          dim3((unsigned)((long long)p.B * p.Hq * nqt)), dim3(256), kargs, 0, stream);
    if (err != hipSuccess) return err;
    const long long nkt = (p.N + 127) / 128;
    p.xcd_map = ((long long)p.B * p.Hkv) % 8 == 0 ? 1 : 0;
    err = hipLaunchKernel(causal ? (const void*)&bwd_dkdv_kernel<E, D, true> : (const void*)&bwd_dkdv_kernel<E, D, false>,
                          dim3((unsigned)((long long)p.B * p.Hkv * nkt * p.splits)), dim3(256), kargs, 0, stream);
    if (err != hipSuccess || p.splits == 1) return err;
    const long long groups = 2LL * p.B * p.Hkv * p.N * D / 8;
    return hipLaunchKernel((const void*)&bwd_reduce_kernel<E, D>, dim3((unsigned)((groups + 255) / 256)), dim3(256),
                           kargs, 0, stream);
}
}  // namespace

hipError_t launch_bwd(const BwdParams& p, int d, int dtype, int causal, hipStream_t stream)
{
    if (dtype == 1) return d == 128 ? launch_bwd_t<__bf16, 128>(p, causal, stream) : launch_bwd_t<__bf16, 64>(p, causal, stream);
    return d == 128 ? launch_bwd_t<_Float16, 128>(p, causal, stream) : launch_bwd_t<_Float16, 64>(p, causal, stream);
}
#endif

}  // namespace fa
