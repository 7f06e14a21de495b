// fa_fwd_w64.hip -- FlashAttention forward for gfx950 (CDNA4, MI355X), 16-bit inputs
// (bf16 or fp16), head dimension 64 or 128: 64 query rows per wave, one wave per SIMD.
//
// Same method and the same per-row arithmetic as fwd16_kernel (fa_fwd_mfma16.hip): the
// online softmax of the pages in base 2 (mbrenndoerfer.com "Online Softmax Computation",
// its update equations; spicyshark.co online-softmax lesson, "The idea", "From softmax to
// attention" and "The implementation"), query blocks outer and key blocks inner (kbwen.com
// FlashAttention feed, "More than two blocks"), with a lazy reference m: it moves only when a
// row maximum has outrun it by more than a slack (bf16: 2^48, fp16: 2^15, so that P stays
// representable; l and O share the stale reference, so u / l is unchanged), and the guard
// for rows with no finite score yet (0 as the exp reference).  P is summed into l in fp32
// before it is rounded to the element type for the PV product.
//
// What differs is the shape of the work.  Each wave owns 64 query rows as two 32-row
// blocks, so every K or V operand read from LDS feeds two matrix products (half the LDS
// reads per flop of a 32-row wave), and runs alone on its SIMD.  A workgroup is 2 waves (128
// rows; two workgroups per CU) or 4 waves (256 rows; one per CU, all four SIMDs), and the
// waves split each tile's loads.  The output accumulators (128 per lane at d = 128) stay in
// AGPRs for the whole key walk, so the register file holds Q, two score buffers and two
// weight buffers beside them.  The key walk runs in 32-key halves of the 64-key LDS tiles;
// in half h a wave issues the score products of half h+1 and the value products of half h-1
// while its vector unit runs the softmax of half h.  That schedule is written out as
// assembly by gen_fwd_kloop.py (fa_fwd_kloop.inc): the compiler would copy the accumulators
// out of the AGPRs for the rare rescale and would not keep the three streams interleaved.
// This file computes the addresses and hands them to that assembly; the assembly loads Q,
// walks the tiles and stores O and LSE.
//
// 256-row workgroups walk pairs of query tiles (the heaviest causal tile of a head with its
// lightest) when that balances as well as one tile per workgroup: one workgroup per CU,
// no dispatch gaps, and every CU gets the same causal work.  Each item (query tile) of the
// walk loads the next one's first K/V tiles and stages its Q rows in LDS during its own last
// two steps, so the next item starts without waiting for memory.
//
// LDS: sets of 4 tiles (64 KiB at d = 128, 32 KiB at d = 64; two sets for 256-row workgroups,
// used by consecutive items in turn): K tiles at +0 and +TILE, V tiles at +2 TILE and
// +3 TILE, each [64 keys][d] with 16-byte chunks XOR-swizzled per row (the layout of
// fa_fwd_mfma16.hip), filled by buffer_load_dwordx4 ... lds.  Rows past N read as zero and
// rows of O and LSE past N are not written: every buffer range ends at the head's last row.
#include "fa_kernels.h"
#include "fa_mfma16_common.h"
#include "fa_fwd_kloop.inc"

#include <float.h>
#include <stdint.h>

namespace fa {

#define FA_W64_CLOBBERS                                                                                   \
    "v0", "v1", "v2", "v3", "v4", "v5", "v6", "v7", "v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15",   \
    "v16", "v17", "v18", "v19", "v20", "v21", "v22", "v23", "v24", "v25", "v26", "v27", "v28", "v29", "v30", \
    "v31", "v32", "v33", "v34", "v35", "v36", "v37", "v38", "v39", "v40", "v41", "v42", "v43", "v44", "v45", \
    "v46", "v47", "v48", "v49", "v50", "v51", "v52", "v53", "v54", "v55", "v56", "v57", "v58", "v59", "v60", \
    "v61", "v62", "v63", "v64", "v65", "v66", "v67", "v68", "v69", "v70", "v71", "v72", "v73", "v74", "v75", \
    "v76", "v77", "v78", "v79", "v80", "v81", "v82", "v83", "v84", "v85", "v86", "v87", "v88", "v89", "v90", \
    "v91", "v92", "v93", "v94", "v95", "v96", "v97", "v98", "v99", "v100", "v101", "v102", "v103", "v104",   \
    "v105", "v106", "v107", "v108", "v109", "v110", "v111", "v112", "v113", "v114", "v115", "v116", "v117",  \
    "v118", "v119", "v120", "v121", "v122", "v123", "v124", "v125", "v126", "v127", "v128", "v129", "v130",  \
    "v131", "v132", "v133", "v134", "v135", "v136", "v137", "v138", "v139", "v140", "v141", "v142", "v143",  \
    "v144", "v145", "v146", "v147", "v148", "v149", "v150", "v151", "v152", "v153", "v154", "v155", "v156",  \
    "v157", "v158", "v159", "v160", "v161", "v162", "v163", "v164", "v165", "v166", "v167", "v168", "v169",  \
    "v170", "v171", "v172", "v173", "v174", "v175", "v176", "v177", "v178", "v179", "v180", "v181", "v182",  \
    "v183", "v184", "v185", "v186", "v187", "v188", "v189", "v190", "v191", "v192", "v193", "v194", "v195",  \
    "v196", "v197", "v198", "v199", "v200", "v201", "v202", "v203", "v204", "v205", "v206", "v207", "v208",  \
    "v209", "v210", "v211", "v212", "v213", "v214", "v215", "v216", "v217", "v218", "v219", "v220", "v221",  \
    "v222", "v223",                                                                                           \
    "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", "a10", "a11", "a12", "a13", "a14", "a15",   \
    "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27", "a28", "a29", "a30", \
    "a31", "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42", "a43", "a44", "a45", \
    "a46", "a47", "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57", "a58", "a59", "a60", \
    "a61", "a62", "a63", "a64", "a65", "a66", "a67", "a68", "a69", "a70", "a71", "a72", "a73", "a74", "a75", \
    "a76", "a77", "a78", "a79", "a80", "a81", "a82", "a83", "a84", "a85", "a86", "a87", "a88", "a89", "a90", \
    "a91", "a92", "a93", "a94", "a95", "a96", "a97", "a98", "a99", "a100", "a101", "a102", "a103", "a104",   \
    "a105", "a106", "a107", "a108", "a109", "a110", "a111", "a112", "a113", "a114", "a115", "a116", "a117",  \
    "a118", "a119", "a120", "a121", "a122", "a123", "a124", "a125", "a126", "a127", "a128", "a129", "a130",  \
    "a131", "a132", "a133", "a134", "a135", "a136", "a137", "a138", "a139", "a140", "a141", "a142", "a143",  \
    "a144", "a145", "a146", "a147", "a148", "a149", "a150", "a151", "a152", "a153", "a154", "a155", "a156",  \
    "a157", "a158", "a159", "vcc", "m0", "scc", "memory"

template <typename E, bool CAUSAL, int NW, int D>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
fwd_w64_kernel(const FwdParams p)
{
    static_assert(NW == 2 || NW == 4, "two or four waves of 64 rows");
    constexpr int R = 64;             // query rows per wave
    static_assert(D == 64 || D == 128, "head dimension 64 or 128");
    constexpr int ROWB = D * 2;
    constexpr int TILE = 64 * ROWB;   // one 64-key K or V tile
    constexpr int BM = R * NW;        // query rows of the workgroup
    constexpr int CPR = ROWB / 16;    // 16-byte chunks per row
    constexpr int RPS = 1024 / ROWB;  // rows per 1 KiB load slice
    // Two sets of four tiles, set s at 4 s TILE: K0, K1, V0, V1 at +0, +TILE, +2 TILE, +3 TILE.
    // Consecutive items of a workgroup use the two sets in turn, so that an item's last steps can
    // load the next item's first tiles.  Aligned to 32 KiB: the walk switches buffers by flipping
    // the TILE bit of the addresses.  128-row workgroups run one item and use the first set.
    constexpr int SETS = NW == 4 ? 2 : 1;
    __shared__ __attribute__((aligned(32768))) char lds[SETS * 4 * TILE];

    const int N = p.N;
    const int units = p.B * p.Hq;
    const int nqt = p.n_qtiles;
    const int bid = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    unsigned long long real0 = 0, cyc0 = 0;
    if (p.stamps) {
        real0 = __builtin_amdgcn_s_memrealtime();
        cyc0 = __builtin_amdgcn_s_memtime();
    }
    // Items: query tiles.  With the walk, the workgroup takes pairs j, j + G, ... of the units *
    // ceil(nqt / 2) pairs; pair j is query tiles nqt - 1 - i and i (i = j mod the pairs per head)
    // of one head, whose causal work adds up to the same for every i.  With the XCD map, logical
    // workgroup ids run down each XCD in turn, so the pairs of a head (and of heads sharing K/V)
    // stay in one L2.  Without the walk, one query tile per workgroup.
    const int per_head = (nqt + 1) >> 1;
    int j = 0, jstep = 1, jend = 1;
    if (p.walk) {
        const int G = gridDim.x;
        j = p.xcd_map ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;
        jstep = G;
        jend = units * per_head;
    }
    auto tile_of = [&](int jj, int ss, int& bh, int& qt) {
        if (p.walk) {
            bh = jj / per_head;
            const int i = jj - bh * per_head;
            qt = ss == 0 ? nqt - 1 - i : i;
        } else if (p.xcd_map) {
            int t;
            xcd_order(bid, units, nqt, bh, t);
            qt = CAUSAL ? nqt - 1 - t : t;   // longest first
        } else {
            bh = bid % units;
            qt = CAUSAL ? nqt - 1 - bid / units : bid / units;
        }
    };
    auto next_of = [&](int& jj, int& ss) {
        if (p.walk && ss == 0) {
            const int i = jj - (jj / per_head) * per_head;
            if (i != nqt - 1 - i) {          // the middle tile of an odd count has no partner
                ss = 1;
                return;
            }
        }
        jj += jstep;
        ss = 0;
    };
    const int range = N * ROWB;
    auto rsrc = [&](const void* base, int bytes) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
    };
    const unsigned ldsb = (unsigned)(uintptr_t)(FA_LDS char*)lds;
    // Tile loads: slice ii = wave + NW i of a tile holds LDS bytes [1024 ii, 1024 ii + 1024); this
    // lane's 16 bytes are row RPS ii + lane / CPR, physical chunk lane % CPR, i.e. logical chunk
    // (lane % CPR) ^ swz(row).  ii enters the swizzle only through ii mod 4 (d = 128) or ii mod 2
    // (d = 64): two patterns (i even, odd; the same one when NW = 4).
    int dma[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int row = RPS * (wave + NW * e) + lane / CPR;
        dma[e] = 1024 * wave + (lane / CPR) * ROWB + 16 * ((lane % CPR) ^ swz<D>(row));
    }
    const int dmask = l32 - 4 * hi;   // causal: key 8(r>>2) + (r&3) + 4hi of a diagonal half visible iff <= row l32
    const int hi4 = 4 * hi;
    // A negative scale is folded into Q's sign; a zero scale becomes the smallest normal.
    const float c = fmaxf(fabsf(p.scale_log2), FLT_MIN);
    const unsigned flip = p.scale_log2 >= 0.f ? 0u : 0x80008000u;
    // Key tiles of 64 that query tile qt visits: up to the end of its last row when causal.
    auto key_tiles = [&](int qt) {
        const int kv_end = CAUSAL ? min(N, qt * BM + BM) : N;
        return (kv_end + 63) / 64;
    };

    int s = 0, set = 0;
    unsigned pf = 0;                 // 1: this item's first tiles and Q were loaded by the item before
    int qlds = 0;                    // then: this lane's 16 bytes of the staged Q
#pragma nounroll
    while (j < jend) {
        int bh, qt;
        tile_of(j, s, bh, qt);
        int jn = j, sn = s;
        next_of(jn, sn);
        const bool has_next = jn < jend;
        int bhn = bh, qtn = qt;
        if (has_next) tile_of(jn, sn, bhn, qtn);

        const int b = bh / p.Hq;
        const int hk = (bh - b * p.Hq) / p.group;
        const char* Kh = (const char*)p.k + (size_t)(b * p.Hkv + hk) * N * ROWB;
        const char* Vh = (const char*)p.v + (size_t)(b * p.Hkv + hk) * N * ROWB;
        const char* Qh = (const char*)p.q + (size_t)bh * N * ROWB;
        char* Oh = (char*)p.o + (size_t)bh * N * ROWB;
        float* Lh = p.lse + (size_t)bh * N;
        const __amdgpu_buffer_rsrc_t krs = rsrc(Kh, range);
        const __amdgpu_buffer_rsrc_t vrs = rsrc(Vh, range);
        const __amdgpu_buffer_rsrc_t qrs = rsrc(Qh, range);
        const __amdgpu_buffer_rsrc_t ors = rsrc(Oh, range);
        const __amdgpu_buffer_rsrc_t lrs = rsrc(Lh, N * 4);
        // the next item's head (its K/V tiles and Q rows are loaded in this item's last steps)
        const int bn = bhn / p.Hq;
        const int hkn = (bhn - bn * p.Hq) / p.group;
        const __amdgpu_buffer_rsrc_t nkrs = rsrc((const char*)p.k + (size_t)(bn * p.Hkv + hkn) * N * ROWB, range);
        const __amdgpu_buffer_rsrc_t nvrs = rsrc((const char*)p.v + (size_t)(bn * p.Hkv + hkn) * N * ROWB, range);
        const __amdgpu_buffer_rsrc_t nqrs = rsrc((const char*)p.q + (size_t)bhn * N * ROWB, range);

        const int q0 = qt * BM;
        const int row0 = q0 + R * wave;                     // the wave's first query row
        const int qoff = (row0 + l32) * ROWB + 16 * hi;      // Q: dims 16kk + 8hi .. of this lane's row
        const int ooff = (row0 + l32) * ROWB + 8 * hi;       // O: dims 32db + 8g + 4hi .. of this lane's row
        const int loff = (row0 + l32) * 4;
        const int nqoff = (qtn * BM + R * wave + l32) * ROWB + 16 * hi;
        const unsigned setb = ldsb + (unsigned)(set * 4 * TILE);
        const unsigned nsetb = ldsb + (unsigned)((set ^ (SETS - 1)) * 4 * TILE);

        // K operand: row l32 of the 32-key block, logical chunk 2kk + hi (buffer K0 to start).
        const int kx = swz<D>(l32);
        int koff[8] = {};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) koff[kk] = (int)setb + l32 * ROWB + 16 * ((2 * kk + hi) ^ kx);
        // V operand (transposed reads): lane (group G, 4j + s) reads row 8r + 4(G>>1) + j of a 16-key
        // step and dims 32dt + 16(G&1) + 4s ..; buffer V0 to start (V tile 0 lands in V1).
        const int G = lane >> 4;
        const int jj = (lane >> 2) & 3;
        const int ss = lane & 3;
        int voff[8] = {};
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = 8 * r + 4 * (G >> 1) + jj;
            const int w = swz<D>(row);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const int chunk = 4 * dt + 2 * (G & 1) + (ss >> 1);
                voff[(D / 32) * r + dt] = (int)setb + 2 * TILE + row * ROWB + 16 * (chunk ^ w) + 8 * (ss & 1);
            }
        }

        // Key tiles of 64 for the workgroup; the last one this wave's rows need.
        const int nt = key_tiles(qt);
        const int last = CAUSAL ? min(nt - 1, (q0 + R * wave) / 64) : nt - 1;
        const int valid_last = N - 64 * (nt - 1);            // keys of the last tile below N (non-causal mask)
        const int limA = valid_last - 1;
        const int limB = valid_last - 33;
        const int nnt = key_tiles(qtn);
        // The next item's loads: its first K/V tiles at step max(nt - 1, 1) into the other set, its
        // Q rows at step nt (no S product of this item follows) into this wave's staging area: the
        // K buffers and the idle V buffer of this set (waves 0-2) or V0 of the other set (wave 3),
        // none of which this item reads after step nt - 1 or the next one fills before its own Q is read.
        const unsigned never = 0xffffffffu;
        const unsigned pkv = has_next ? (unsigned)max(nt - 1, 1) : never;
        const unsigned pq = has_next ? (unsigned)nt : never;
        const unsigned nkdst = nsetb + 1024 * wave;
        unsigned qst;
        if (wave == 0) qst = setb;
        else if (wave == 1) qst = setb + TILE;
        else if (wave == 2) qst = setb + 2 * TILE + ((nt + 1) & 1) * TILE;
        else qst = nsetb + 2 * TILE;
        const int qlds_next = (int)qst + 16 * lane;

        // K tile j lands in K buffer j % 2, V tile j in V buffer (j + 1) % 2; the operand reads
        // start at buffer 0 of each and flip before every tile (V tile j is read one tile later)
        unsigned ksrc = 0, kdst = setb + 1024 * wave, vsrc = 0, vdst = setb + 3 * TILE + 1024 * wave;
        unsigned soff, kit, cnt;
        unsigned long long g00, g01, g10, g11, ga0, ga1, mk1, mk2, mk3, mk4, mk5, mk6, mk7;
        int dlim;
#define FA_W64_ASM_C(TEXT, CLOBBERS)                                                                       \
        asm volatile(TEXT                                                                                      \
                     : [koff0] "+v"(koff[0]), [koff1] "+v"(koff[1]), [koff2] "+v"(koff[2]), [koff3] "+v"(koff[3]),  \
                       [koff4] "+v"(koff[4]), [koff5] "+v"(koff[5]), [koff6] "+v"(koff[6]), [koff7] "+v"(koff[7]),  \
                       [voff0] "+v"(voff[0]), [voff1] "+v"(voff[1]), [voff2] "+v"(voff[2]), [voff3] "+v"(voff[3]),  \
                       [voff4] "+v"(voff[4]), [voff5] "+v"(voff[5]), [voff6] "+v"(voff[6]), [voff7] "+v"(voff[7]),  \
                       [ksrc] "+s"(ksrc), [kdst] "+s"(kdst), [vsrc] "+s"(vsrc), [vdst] "+s"(vdst),                   \
                       [soff] "=&s"(soff), [kit] "=&s"(kit), [cnt] "=&s"(cnt),                                      \
                       [g00] "=&s"(g00), [g01] "=&s"(g01), [g10] "=&s"(g10), [g11] "=&s"(g11), [ga0] "=&s"(ga0),    \
                       [ga1] "=&s"(ga1), [mk1] "=&s"(mk1), [mk2] "=&s"(mk2), [mk3] "=&s"(mk3), [mk4] "=&s"(mk4),    \
                       [mk5] "=&s"(mk5), [mk6] "=&s"(mk6), [mk7] "=&s"(mk7), [dlim] "=&v"(dlim)                     \
                     : [dma0] "v"(dma[0]), [dma1] "v"(dma[1]), [qoff] "v"(qoff), [ooff] "v"(ooff), [loff] "v"(loff),  \
                       [dmask] "v"(dmask), [hi4] "v"(hi4), [krs] "s"(krs), [vrs] "s"(vrs), [qrs] "s"(qrs),             \
                       [ors] "s"(ors), [lrs] "s"(lrs), [nt] "s"(nt), [last] "s"(last), [limA] "s"(limA),              \
                       [limB] "s"(limB), [c] "s"(c), [flip] "s"(flip), [pf] "s"(pf), [qlds] "v"(qlds),               \
                       [pkv] "s"(pkv), [pq] "s"(pq), [nkrs] "s"(nkrs), [nvrs] "s"(nvrs), [nqrs] "s"(nqrs),            \
                       [nqoff] "v"(nqoff), [nkdst] "s"(nkdst), [nnt] "s"(nnt), [qst] "s"(qst)                        \
                     : CLOBBERS)
#define FA_W64_ASM(TEXT) FA_W64_ASM_C(TEXT, FA_W64_CLOBBERS)
#define FA_W64_PICK(W, DD)                                                                 \
        if constexpr (__is_same(E, __bf16)) {                                                 \
            if constexpr (CAUSAL) FA_W64_ASM(FA_KLOOP_BF16_CAUSAL_W##W##_D##DD);              \
            else FA_W64_ASM(FA_KLOOP_BF16_FULL_W##W##_D##DD);                                 \
        } else {                                                                              \
            if constexpr (CAUSAL) FA_W64_ASM(FA_KLOOP_F16_CAUSAL_W##W##_D##DD);               \
            else FA_W64_ASM(FA_KLOOP_F16_FULL_W##W##_D##DD);                                  \
        }
        if constexpr (D == 128) {
            if constexpr (NW == 2) {
                FA_W64_PICK(2, 128)
            } else {
                FA_W64_PICK(4, 128)
            }
        } else {
            if constexpr (NW == 2) {
                FA_W64_PICK(2, 64)
            } else {
                FA_W64_PICK(4, 64)
            }
        }
#undef FA_W64_PICK
#undef FA_W64_ASM
#undef FA_W64_ASM_C
        // No barrier here: the next item's first barrier comes before anything it writes to LDS
        // could reach a tile this item still reads.
        j = jn;
        s = sn;
        set ^= SETS - 1;
        pf = 1;
        qlds = qlds_next;
    }

    if (p.stamps && lane == 0) {
        const unsigned long long cyc1 = __builtin_amdgcn_s_memtime();
        const unsigned long long real1 = __builtin_amdgcn_s_memrealtime();
        typedef __attribute__((ext_vector_type(4))) unsigned long long u64x4;
        *(u64x4*)(p.stamps + ((size_t)bid * NW + wave) * 4) = u64x4{real0, real1, cyc0, cyc1};
    }
}

#define FA_W64_INSTANTIATE(NW, DD)                                                      \
    template __global__ void fwd_w64_kernel<__bf16, false, NW, DD>(const FwdParams);   \
    template __global__ void fwd_w64_kernel<__bf16, true, NW, DD>(const FwdParams);    \
    template __global__ void fwd_w64_kernel<_Float16, false, NW, DD>(const FwdParams); \
    template __global__ void fwd_w64_kernel<_Float16, true, NW, DD>(const FwdParams);
FA_W64_INSTANTIATE(2, 128)
FA_W64_INSTANTIATE(4, 128)
FA_W64_INSTANTIATE(2, 64)
FA_W64_INSTANTIATE(4, 64)

#if !defined(__HIP_DEVICE_COMPILE__)
namespace {

// 256-row workgroups walk pairs of query tiles: one workgroup per CU at most (each holds a
// whole CU: one wave per SIMD), as many as give every workgroup the same number of pairs, a
// multiple of 8 (whole groups of the XCD map).  0 (one tile per workgroup) when the tiles fit
// on the CUs at once, or when whole pairs would balance worse than single tiles: the walk's
// critical path is its rounds of pairs (a causal pair is ntiles + 1 tile-rows of work, a
// non-causal one two tiles), the other's the larger of an even share and the largest tile.
long long w64_walk_blocks(long long units, long long ntiles, int causal)
{
    const int cus = device_cus();
    if (cus <= 0 || units * ntiles <= cus) return 0;
    const long long pairs = units * ((ntiles + 1) / 2);
    const long long rounds = (pairs + cus - 1) / cus;
    double walk, tiles;
    if (causal) {
        walk = (double)rounds * (double)(ntiles + 1);
        tiles = (double)units * (double)ntiles * (double)(ntiles + 1) / 2.0 / cus;
        if (tiles < (double)ntiles) tiles = (double)ntiles;
    } else {
        walk = 2.0 * (double)rounds;
        tiles = (double)((units * ntiles + cus - 1) / cus);
    }
    if (walk > 1.03 * tiles) return 0;
    long long g = (pairs + rounds - 1) / rounds;
    if (cus % 8 == 0) g = (g + 7) / 8 * 8;
    return g;
}

template <typename E, bool CAUSAL, int NW, int D>
hipError_t launch_w64(const FwdParams& p, hipStream_t stream)
{
    const long long units = (long long)p.B * p.Hq;
    FwdParams args = p;
    long long grid = units * p.n_qtiles;
    const long long walk = NW == 4 ? w64_walk_blocks(units, p.n_qtiles, CAUSAL) : 0;
    if (walk > 0) {
        grid = walk;
        args.walk = 1;
        args.xcd_map = (walk % 8 == 0) ? 1 : 0;
    } else {
        args.walk = 0;
        args.xcd_map = (units % 8 == 0) ? 1 : 0;   // needs whole heads per XCD
    }
    void* kargs[] = {&args};
    return hipLaunchKernel((const void*)&fwd_w64_kernel<E, CAUSAL, NW, D>, dim3((unsigned)grid), dim3(64 * NW),
                           kargs, 0, stream);
}

}  // namespace

// 256-row workgroups first: one K/V tile load per CU instead of two (2-3% faster on the causal
// d = 128 workloads); the host falls back to 128-row workgroups for grids too small to give
// every CU two of them.
#define FA_W64_ENTRIES(CODE, E, DD)                                                             \
    {CODE, DD, 256, 64, 0, &launch_w64<E, false, 4, DD>, 4, &w64_walk_blocks},                  \
        {CODE, DD, 256, 64, 1, &launch_w64<E, true, 4, DD>, 4, &w64_walk_blocks},               \
        {CODE, DD, 128, 64, 0, &launch_w64<E, false, 2, DD>, 2, nullptr},                       \
        {CODE, DD, 128, 64, 1, &launch_w64<E, true, 2, DD>, 2, nullptr}
const KernelEntry kBf16W64Kernels[] = {FA_W64_ENTRIES(1, __bf16, 128), FA_W64_ENTRIES(1, __bf16, 64)};
const KernelEntry kF16W64Kernels[] = {FA_W64_ENTRIES(2, _Float16, 128), FA_W64_ENTRIES(2, _Float16, 64)};
#undef FA_W64_ENTRIES
#endif

}  // namespace fa
