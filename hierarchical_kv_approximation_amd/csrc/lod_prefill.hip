// lod_prefill.hip -- LoD prefill (causal, many query rows per call) and the dense
// causal prefill baseline, on MFMA.
//
// Every query row p computes what a decode query at p computes ("Level of Detail
// Attention", How It Works): top groups by centroid score, top pages inside them, exact
// attention over opened pages, the block window and the sinks, and the coarse remainder,
// all in one softmax.  The rows of a 256-token chunk share the summarised chunks, so the
// work is organised around tiles of 128 (query row, head) pairs of one KV head:
//
//   select   per tile: two MFMA sweeps over the group centroids find, for every
//            (row, head), the k-th largest lower bound of the MFMA score and the groups
//            whose upper bound reaches it; those are re-scored with the canonical fp32
//            chain and ranked exactly; then the pages of the opened groups are ranked.
//   flash    per tile: one online softmax over the coarse centroids (bias ln n, the
//            row's opened groups masked out), the sinks and the causal block window.
//   bucket   per (query chunk, KV head): the (row, head, opened slot) pairs sorted by
//            opened group.
//   pages    per run of pairs that opened the same group (MFMA): the group's members and
//            page summaries are one key tile shared by those pairs, each pair a column
//            with its page mask: exact rows of opened pages, mean terms of unopened ones.
//   combine  per (row, head): log-sum-exp merge of the flash and page partial states.
// Every kernel of a call runs on the caller's stream, one after another.
//
// The flash kernel keeps keys as MFMA rows and (row, head) pairs as MFMA columns
// (S^T = K Q^T), so a lane holds one column of P and the PV product O^T = V^T P^T takes
// P straight from registers; V is staged transposed in LDS.  P enters the PV MFMA as
// bf16 hi + lo parts (error below 2^-16 relative).
#include <climits>

#include "lod_mfma.h"

namespace lodi {

__device__ __forceinline__ int nbuilt_prefill(int p, int W) {
    const int nb = p / kChunk - W / kChunk + 1;
    return nb < 0 ? 0 : nb;
}

struct FlashArgs {
    const bf16_t* k;
    const bf16_t* v;
    int64_t sb, st, sh;
    const int32_t* btab;  // paged view: block table [batch][maxb], else null
    int bshift, maxb;
    const bf16_t* q;  // rows of this launch: [B][nq][Hq][d]
    int seq;          // sequence of grid slice z = 0 (index and cache)
    int nq;           // rows per sequence in this launch
    int pos0;         // position of row 0
    int Hq, Hkv;
    float scale;
    // LoD sources; index == nullptr selects the dense causal mode
    const char* index;
    lod_index_layout_t L;
    int max_chunks, G, W, n_sink, TG;
    int drop;             // LoD: 1 = no coarse remainder (sparsity ablation)
    const int32_t* selg;  // [B][nq][Hq][TG] opened groups sorted ascending, -1 padding
    float* part;          // LoD: [nsplit][B][nq][Hq] partial states (o[d], m, l)
    int nsplit;           // LoD: workgroups sharing one tile's key list
    int64_t split_stride; // floats between the partial arrays of two splits
    float* out;           // dense: normalised output [B][nq][Hq][d]
};

// K and V tiles are double buffered and loaded straight into LDS; both are row-major
// with 16-byte chunks XOR-swizzled (K by row & 15, V by 2 (row & 7), so the 16 rows a
// transposing read touches fall on distinct banks); V^T operands come from gfx950's
// transposing LDS read.  Logits are kept in log2 units (exp2 weights); a partial
// state's maximum is written back in natural units.
template <int HG>
struct FlashSmem {
    alignas(16) bf16_t kt[2][kFlashKeys][kD];  // key tiles (double buffer)
    alignas(16) bf16_t vt[2][kFlashKeys][kD];  // value tiles (double buffer)
    alignas(16) float bias[2][kFlashKeys];     // log2 units; -inf: not a key
    alignas(16) float lnr[2][kFlashKeys];      // ln n of a coarse tile's centroids, as loaded
    int32_t sel[kFlashRowHeads][kMaxTG];       // opened groups per column (LoD)
};

constexpr float kFlashLog2e = 1.4426950408889634f;
constexpr float kFlashLn2 = 0.6931471805599453f;

__device__ __forceinline__ int fswz_k(int row) { return row & 15; }
__device__ __forceinline__ int fswz_v(int row) { return 2 * (row & 7); }

typedef short fs16x4_t __attribute__((ext_vector_type(4)));
typedef float ff32x2_t __attribute__((ext_vector_type(2)));
typedef float ff32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 fbf16x2_t __attribute__((ext_vector_type(2)));

// 4 bf16 of a V^T operand: this lane gets V[key0 + r][d0 + lane % 16] for r = 0..3,
// where the 16 lanes of its group read (row key0 + i / 4, elements d0 + 4 (i % 4) ..).
__device__ __forceinline__ fs16x4_t flash_vt_read(const bf16_t (*vt)[kD], int key0, int d0, int i) {
    const int row = key0 + (i >> 2);
    const int e = d0 + 4 * (i & 3);
    const int chunk = (e >> 3) ^ fswz_v(row);
    const bf16_t* p = &vt[row][8 * chunk + (e & 7)];
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) fs16x4_t*)(p));
}

// Load key tile (coarse, k0, nk) into buffer buf: the K and V rows straight into LDS (a
// wave's 64 lanes fill four rows per instruction; rows past nk repeat the last key), and
// for a coarse tile its ln n values, also straight into LDS.  The tile's bias is formed
// from them by flash_commit after the current tile's work: reading
// ln n into a register here made wave 0 wait for that load (and for every load issued
// before it) ahead of its share of the current tile, and the other waves then waited for
// wave 0 at the next barrier.  kb, vb: the rows' base (index summaries for a coarse
// tile, else the cache of this head and sequence).
template <int HG, bool PAGED>
__device__ __forceinline__ void flash_issue(FlashSmem<HG>& s, const FlashArgs& A, int buf, int coarse, int k0, int nk,
                                            const bf16_t* kb, const bf16_t* vb, const float* gln, int bs) {
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
    // every row's offset first (a paged view reads its block table), then the loads: a
    // load whose address waits on a block-table read would wait for the rows before it
    constexpr int kSteps = kFlashKeys / 4 / kFlashWaves;
    int64_t off[kSteps];
#pragma unroll
    for (int ii = 0; ii < kSteps; ++ii) {
        const int row = 4 * (w + kFlashWaves * ii) + g;
        const int rr = row < nk ? row : nk - 1;
        off[ii] = coarse ? (int64_t)(k0 + rr) * kD : kv_pos<PAGED>(A, bs, k0 + rr);
    }
#pragma unroll
    for (int ii = 0; ii < kSteps; ++ii) {
        const int i = w + kFlashWaves * ii;
        const int row = 4 * i + g;
        __builtin_amdgcn_global_load_lds(kb + off[ii] + 8 * (li ^ fswz_k(row)), &s.kt[buf][4 * i][0], 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vb + off[ii] + 8 * (li ^ fswz_v(row)), &s.vt[buf][4 * i][0], 16, 0, 0);
    }
    // lane l's value lands at lnr[buf][l] (keys past nk repeat the last one)
    if (tid < kFlashKeys && coarse)
        __builtin_amdgcn_global_load_lds(gln + k0 + min(l, nk - 1), &s.lnr[buf][0], 4, 0, 0);
}

// The tile's bias (log2 units; -inf: not a key) into buffer buf, by wave 0 once its loads
// have landed.
template <int HG>
__device__ __forceinline__ void flash_commit(FlashSmem<HG>& s, int buf, int coarse, int nk) {
    if (threadIdx.x < kFlashKeys) {
        // the lane index through empty asm: its LDS addresses are formed here, not kept
        // in registers across the tile loop
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): ln n in LDS
        const bool in = tid < nk;
        s.bias[buf][tid] = in ? (coarse ? s.lnr[buf][tid] * kFlashLog2e : 0.0f) : -INFINITY;
    }
}

// Workgroup: 128 (row, head) columns = (128 / HG) query rows x HG heads of one KV head,
// in 8 waves.  Column n = row * HG + head; wave w owns column block w (columns 16w ..
// 16w+15), so a wave's registers stay under 128 and four waves share each SIMD: with
// two column blocks per wave (4 waves, 232 registers) only two did, and the softmax and
// conversion chains left the matrix cores idle four fifths of the time.
// lin: the workgroup's index in the (x, y) plane of the flash grid.
template <int HG, bool PAGED>
__device__ __forceinline__ void flash_body(const FlashArgs& A, FlashSmem<HG>& s, int lin) {
    constexpr int QT = kFlashRowHeads / HG;
    const int nsplit = A.index ? A.nsplit : 1;
    // KV head fastest in the workgroup order: workgroups go to the 8 XCDs round robin, so
    // each XCD's L2 serves the key tiles of one KV head (with the tile fastest, every
    // XCD streamed every head's centroids)
    const int kvh = lin % A.Hkv, tx = lin / A.Hkv;
    const int tile = tx / nsplit, split = tx % nsplit;
    const int b = blockIdx.z, bs = A.seq + b;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
    const int r0 = tile * QT;
    const int nrows = min(QT, A.nq - r0);
    const int p_first = A.pos0 + r0, p_last = A.pos0 + r0 + nrows - 1;
    const int hq0 = kvh * HG;
    const float sc2 = A.scale * kFlashLog2e;

    // Q^T operands for this lane's column, its row position
    bf16x8_t qb[4];
    int prow, colrow;
    {
        const int n = 16 * w + li;
        const int rl = n / HG, h = n % HG;
        colrow = rl;
        prow = rl < nrows ? A.pos0 + r0 + rl : -1;  // -1: no cache key passes
        const bf16_t* qr = A.q + (((int64_t)b * A.nq + r0 + min(rl, nrows - 1)) * A.Hq + hq0 + h) * kD;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qb[kk] = *reinterpret_cast<const bf16x8_t*>(qr + 32 * kk + 8 * g);
    }
    f32x4_t O[8];
    float m_run = -INFINITY, l_run = 0.0f;
#pragma unroll
    for (int db = 0; db < 8; ++db) O[db] = {0.0f, 0.0f, 0.0f, 0.0f};
    // head kvh of sequence bs; the row of position x adds kv_pos(A, bs, x)
    const bf16_t* kc = A.k + kvh * A.sh + kv_seq<PAGED>(A, bs);
    const bf16_t* vc = A.v + kvh * A.sh + kv_seq<PAGED>(A, bs);

    // Key tiles.  Dense causal: keys [0, p_last] in tiles of 64.  LoD: coarse centroids
    // (bias ln n, each column's opened groups masked), then the sinks, then the causal
    // block window [nb*C, p]; split `split` of `nsplit` takes an equal share of the list.
    int ct = 0, st = 0, ng = 0, ns = 0, w0 = 0, nt, t0 = 0, t1;
    const bf16_t* gk = nullptr;
    const bf16_t* gv = nullptr;
    const float* gln = nullptr;
    if (A.index == nullptr) {
        nt = (p_last + kFlashKeys) / kFlashKeys;
        t1 = nt;
    } else {
        const int nb = nbuilt_prefill(p_first, A.W);
        ng = nb * A.G;
        ns = min(A.n_sink, nb * kChunk);
        w0 = nb * kChunk;
        ct = A.drop ? 0 : (ng + kFlashKeys - 1) / kFlashKeys;  // no remainder: no centroids
        st = (ns + kFlashKeys - 1) / kFlashKeys;
        const int wt = p_last >= w0 ? (p_last - w0) / kFlashKeys + 1 : 0;
        nt = ct + st + wt;
        t0 = split * nt / nsplit;
        t1 = (split + 1) * nt / nsplit;
        const int64_t gbase = ((int64_t)bs * A.Hkv + kvh) * A.max_chunks * A.G;
        gk = reinterpret_cast<const bf16_t*>(A.index + A.L.gk) + gbase * kD;
        gv = reinterpret_cast<const bf16_t*>(A.index + A.L.gv) + gbase * kD;
        gln = reinterpret_cast<const float*>(A.index + A.L.gln) + gbase;
        if (t0 < ct) {
            // opened groups of the tile's columns (left out of the coarse terms)
            for (int x = tid; x < kFlashRowHeads * A.TG; x += kFlashThreads) {
                const int n = x / A.TG, t = x % A.TG;
                const int rl = n / HG, h = n % HG;
                s.sel[n][t] = rl < nrows ? A.selg[(((int64_t)b * A.nq + r0 + rl) * A.Hq + hq0 + h) * A.TG + t] : -1;
            }
            __syncthreads();
        }
    }
    // tile t: kind (0 coarse, 1 sinks / window / dense run), first key, key count
    auto tile_of = [&](int t, int& coarse, int& k0, int& nk) {
        if (A.index == nullptr) {
            coarse = 0;
            k0 = t * kFlashKeys;
            nk = min(kFlashKeys, p_last + 1 - k0);
        } else if (t < ct) {
            coarse = 1;
            k0 = t * kFlashKeys;
            nk = min(kFlashKeys, ng - k0);
        } else if (t < ct + st) {
            coarse = 0;
            k0 = (t - ct) * kFlashKeys;
            nk = min(kFlashKeys, ns - k0);
        } else {
            coarse = 0;
            k0 = w0 + (t - ct - st) * kFlashKeys;
            nk = min(kFlashKeys, p_last + 1 - k0);
        }
    };
    if (t0 < t1) {
        int coarse, k0, nk;
        tile_of(t0, coarse, k0, nk);
        flash_issue<HG, PAGED>(s, A, 0, coarse, k0, nk, coarse ? gk : kc, coarse ? gv : vc, gln, bs);
        flash_commit<HG>(s, 0, coarse, nk);
    }
    int eptr = 0;  // next opened group of this lane's column not yet below the tiles
    for (int t = t0; t < t1; ++t) {
        const int buf = (t - t0) & 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        int coarse, k0, nk;
        if (t + 1 < t1) {
            tile_of(t + 1, coarse, k0, nk);
            flash_issue<HG, PAGED>(s, A, buf ^ 1, coarse, k0, nk, coarse ? gk : kc, coarse ? gv : vc, gln, bs);
        }
        tile_of(t, coarse, k0, nk);
        // excluded keys of this lane's column: its opened groups inside a coarse tile.  The
        // column's list is ascending (-1 after the last) and coarse tiles come in key
        // order, so a pointer that only moves forward visits each opened group once.
        // Only the 16 keys this lane scores are kept: bit 4 kb + r stands for key
        // 16 kb + 4 g + r, so each test below is against a constant bit (a 64-bit mask
        // tested at 16 key positions kept 16 shifted 64-bit constants in registers).
        uint32_t ex = 0;
        if (coarse) {
            const int n = 16 * w + li;
            int gsel;
            while (eptr < A.TG && (gsel = s.sel[n][eptr]) >= 0 && gsel < k0 + kFlashKeys) {
                const int key = gsel - k0;
                if (key >= 0 && ((key >> 2) & 3) == g) ex |= 1u << (4 * (key >> 4) + (key & 3));
                ++eptr;
            }
        }
        // S^T = K Q^T for 4 key blocks.  LDS addresses are formed here from one lane value
        // that the compiler cannot see through, so they are not hoisted out of the loop
        // into registers of their own (a key row 16 kb + li holds chunk 4 kk + g at
        // position (4 kk + g) ^ li)
        int lo_ = li;
        asm volatile("" : "+v"(lo_));
        const bf16_t* ktb = &s.kt[buf][0][0] + lo_ * kD;
        f32x4_t S[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            S[kb] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ktb + 16 * kb * kD + 8 * ((4 * kk + g) ^ lo_));
                S[kb] = mfma16(a, qb[kk], S[kb]);
            }
        }
        // logits (log2 units), masks, online softmax (a column's 64 keys live in lanes
        // l, l^16, l^32, l^48).  A column may see no key in a tile (all masked): its
        // maximum then stays -inf and the guards below keep every weight 0.  The lane's
        // keys 16 kb + 4 g .. 16 kb + 4 g + 3 are consecutive, so their biases come in four
        // 16-byte reads, issued together and waited for once (through empty asm, so no
        // read is sunk into the mask's branch, where each was waited for alone).
        ff32x4_t b4[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) b4[kb] = *reinterpret_cast<const ff32x4_t*>(&s.bias[buf][16 * kb + 4 * g]);
        asm volatile("" : "+v"(b4[0]), "+v"(b4[1]), "+v"(b4[2]), "+v"(b4[3]));
        // keep mask: bit 4 kb + r is set when the lane's key 16 kb + 4 g + r counts.  Coarse
        // tiles: every centroid but the column's opened groups.  Cache tiles: the causal
        // test, key k0 + c visible when c <= prow - k0.  A key that fails gets the bit
        // pattern of -inf through a sign-extended bit field and a bitwise select, two
        // instructions per key.
        uint32_t vm;
        if (coarse) {
            vm = ~ex;
        } else {
            const int d = prow - k0 - 4 * g;  // the lane's key 16 kb + r passes when 16 kb + r <= d
            vm = 0;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int n = min(max(d - 16 * kb + 1, 0), 4);
                vm |= ((1u << n) - 1u) << (4 * kb);
            }
        }
        float P[4][4];
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int keep = __builtin_amdgcn_sbfe((int)vm, 4 * kb + r, 1);  // 0 or -1
                const int lb = __float_as_int(__builtin_fmaf(sc2, S[kb][r], b4[kb][r]));
                const float lam = __int_as_float((lb & keep) | ((int)0xFF800000 & ~keep));  // else -inf
                P[kb][r] = lam;
                mt = fmaxf(mt, lam);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float mn = fmaxf(m_run, mt);
        const float a = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mn);
        const float ms = mn == -INFINITY ? 0.0f : mn;
        float ls = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(P[kb][r] - ms);  // exp2(-inf) = 0
                P[kb][r] = p;
                ls += p;
            }
        l_run = __builtin_fmaf(l_run, a, ls);
        m_run = mn;
        if (__any(a != 1.0f)) {  // the maximum moved for some column of the wave
#pragma unroll
            for (int db = 0; db < 8; ++db) O[db] *= a;
        }
        // O^T += V^T P^T over two 32-key steps.  MFMA k index e of lane group g is key
        // 32 st + 16 (e / 4) + 4 g + e % 4 on both operands; P as bf16 hi + lo.
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            bf16x8_t ph, pl;
#pragma unroll
            for (int j = 0; j < 8; j += 2) {  // two at a time: one packed conversion each
                const ff32x2_t x = {P[2 * sp + j / 4][j % 4], P[2 * sp + j / 4][j % 4 + 1]};
                const fbf16x2_t h = __builtin_convertvector(x, fbf16x2_t);
                const ff32x2_t r = x - __builtin_convertvector(h, ff32x2_t);
                const fbf16x2_t lo = __builtin_convertvector(r, fbf16x2_t);
                ph[j] = h[0];
                ph[j + 1] = h[1];
                pl[j] = lo[0];
                pl[j + 1] = lo[1];
            }
            // V^T operands (flash_vt_read's addresses, formed here as for K): row
            // 32 sp + 4 g + li / 4 (and 16 rows on), elements 16 db + 4 (li % 4) .. at chunk
            // (2 db + (li / 2) % 2) ^ 2 ((4 g + li / 4) % 8)
            int vs_ = 2 * ((4 * g + (li >> 2)) & 7);
            asm volatile("" : "+v"(vs_));
            const bf16_t* vtb = &s.vt[buf][0][0] + (32 * sp + 4 * g + (li >> 2)) * kD + 4 * (li & 1);
            const int vx = (li >> 1) & 1;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const bf16_t* p0 = vtb + 8 * (((2 * db) ^ vs_) + vx);
                typedef __attribute__((address_space(3))) fs16x4_t lds_fs16x4_t;
                const fs16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_fs16x4_t*)(p0));
                const fs16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_fs16x4_t*)(p0 + 16 * kD));
                const fs16x4_t both[2] = {v0, v1};
                const bf16x8_t av = __builtin_bit_cast(bf16x8_t, both);
                O[db] = mfma16(av, ph, O[db]);
                O[db] = mfma16(av, pl, O[db]);
            }
        }
        // buffer buf ^ 1 held tile t - 1, which every wave finished before this tile's barrier
        if (t + 1 < t1) {
            tile_of(t + 1, coarse, k0, nk);
            flash_commit<HG>(s, buf ^ 1, coarse, nk);
        }
    }

    // column total (the 4 lanes of a column hold partial sums), then write
    float lt = l_run;
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int rl = colrow;
    if (rl < nrows) {
        const int n = 16 * w + li;
        const int h = n % HG;
        const int64_t rh = ((int64_t)b * A.nq + r0 + rl) * A.Hq + hq0 + h;
        if (A.index == nullptr) {
            float* dst = A.out + rh * kD;
            const float inv = 1.0f / lt;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const f32x4_t o = O[db];
                *reinterpret_cast<float4*>(dst + 16 * db + 4 * g) =
                    make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
            }
        } else {
            float* dst = A.part + split * A.split_stride + rh * kPartStride;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const f32x4_t o = O[db];
                *reinterpret_cast<float4*>(dst + 16 * db + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
            }
            if (g == 0) {
                dst[kD] = m_run == -INFINITY ? -INFINITY : m_run * kFlashLn2;  // natural units
                dst[kD + 1] = lt;
            }
        }
    }
}

template <int HG, bool PAGED>
__global__ __launch_bounds__(kFlashThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void prefill_flash_kernel(FlashArgs A) {
    __shared__ FlashSmem<HG> s;
    flash_body<HG, PAGED>(A, s, blockIdx.x + gridDim.x * blockIdx.y);
}

}  // namespace lodi

namespace lodi {

// ---------------------------------------------------------------------------- select

// Per (row, head, opened slot) record handed from select to the pages kernel.
struct PairRec {
    int32_t gid;       // opened group c*G + j, -1: none
    int16_t ps0, npg;  // first page slot of the group, number of pages
    uint32_t open;     // bit e: page ps0 + e is opened (exact)
    float r[kPage];    // canonical ranking score of every page (coarse logits of unopened pages)
};

struct SelArgs {
    const bf16_t* q;  // rows of this launch: [B][nq][Hq][d]
    int seq;          // sequence of grid slice z = 0 (index and cache)
    int nq, pos0, Hq, Hkv;
    const char* index;
    lod_index_layout_t L;
    int max_chunks, G, W, TG, TP;
    int nsplit;           // candidate sweeps per tile of columns, each over 1/nsplit of the centroids
    float* ltop;          // [cols][nsplit][kMaxTG] per sweep: its TG largest lower bounds, descending
    int32_t* lcnt;        // [cols][nsplit] per sweep: candidates found (may exceed kSplitCap)
    uint2* lent;          // [cols][nsplit][kSplitCap] per sweep: (group id, upper bound bits)
    int32_t* sel_groups;  // nullable API output [B][nq][Hq][TG], rank order
    int32_t* sel_pages;   // nullable API output [B][nq][Hq][TG][max(TP,1)]
    int32_t* selg;        // [B][nq][Hq][TG] opened groups in ascending id order (-1 pad)
    PairRec* rec;         // [B][nq][Hq][TG] in ascending group order (as selg)
    float* part_pg;       // [B][nq][Hq][TG] page partial states: m = -inf written for empty slots
};

constexpr int kCandCap = 2 * kMaxTG;   // candidates kept per column; beyond: exhaustive path
constexpr int kSplitCap = 2 * kMaxTG;  // candidates kept per column and sweep

// Grid slot -> (tile of columns, split, KV head).  Workgroups are handed to the eight XCDs
// in turn by linear id, so the KV head varies fastest: with eight KV heads each XCD (and
// its L2) serves the centroids of one head.
struct SelSlot {
    int tile, split, kvh;
};
__device__ __forceinline__ SelSlot sel_slot(int Hkv, int nsplit) {
    const int j = blockIdx.x + gridDim.x * blockIdx.y;
    const int rest = j / Hkv;
    return {rest / nsplit, rest % nsplit, j - rest * Hkv};
}

struct CandSmem {
    alignas(16) bf16_t kt[2][kFlashKeys][kD];  // double-buffered centroid tiles
    alignas(16) float gkn_t[2][kFlashKeys];
    alignas(16) float gln_t[2][kFlashKeys];
    float qn[kFlashRowHeads];
    float T[kFlashRowHeads];
    int cnt[kFlashRowHeads];
};

// Canonical ranking chain q . kbar (fp32 fma in index order) for bf16 rows.
// (Loaded 32 elements at a time, with a compiler barrier between the pieces: loading
// both rows whole kept 128 registers live and held the select kernel at two waves per
// SIMD.  The chain's order, and so its result, is unchanged.)
__device__ __forceinline__ float canonical_dot_bf16(const bf16_t* q, const bf16_t* k) {
    float acc = 0.0f;
#pragma unroll
    for (int p4 = 0; p4 < 4; ++p4) {
        uint4 qu[4], ku[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            qu[c] = *reinterpret_cast<const uint4*>(q + 32 * p4 + 8 * c);
            ku[c] = *reinterpret_cast<const uint4*>(k + 32 * p4 + 8 * c);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float qf[8], kf[8];
            Elt<bf16_t>::unpack(qu[c], qf);
            Elt<bf16_t>::unpack(ku[c], kf);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(qf[e], kf[e], acc);
        }
        asm volatile("" ::: "memory");
    }
    return acc;
}

// Stage a 64-row tile of bf16 rows (row stride kD) into LDS with XOR-swizzled chunks.
__device__ __forceinline__ void stage_rows_swizzled(bf16_t (*kt)[kD], const bf16_t* base, int nk) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    for (int i = w; i < kFlashKeys / 4; i += 4) {
        const int row = 4 * i + (l >> 4);
        const int c = (l & 15) ^ (row & 15);
        const int rr = row < nk ? row : nk - 1;
        __builtin_amdgcn_global_load_lds(base + (int64_t)rr * kD + 8 * c, &kt[4 * i][0], 16, 0, 0);
    }
}

// Candidate sweep of one split of the centroid tiles for 128 (row, head) columns.
//
// Group selection opens the TG groups with the largest q . kbar (ties to the lower id)
// under the canonical chain.  The MFMA score S of a group is within
// E = kErrC |q| |kbar| of that chain, so with T the TG-th largest lower bound S - E over
// the groups, the groups with S + E >= T contain the exact top TG; so does any T below
// that one.  Each split keeps, per column, the R largest of the lower bounds' maxima over
// the 4-key blocks seen by each of the column's four lanes (4R >= TG values of distinct
// groups), lists the TG largest of
// those, and collects the groups with S + E at or above the TG-th (a lower bound of the
// split's TG-th largest, never above the global one).  The select step takes the global
// threshold from the splits' top lists and keeps the listed groups at or above it.
template <int HG, int R, bool WT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WT ? 2 : 4, 8)))
void prefill_cand_kernel(SelArgs A) {
    __shared__ CandSmem s;
    constexpr int QT = kFlashRowHeads / HG;
    const SelSlot slot = sel_slot(A.Hkv, A.nsplit);
    const int tile = slot.tile, split = slot.split, kvh = slot.kvh, b = blockIdx.z, bs = A.seq + b;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int r0 = tile * QT;
    const int nrows = min(QT, A.nq - r0);
    const int hq0 = kvh * HG;
    const int nb = nbuilt_prefill(A.pos0 + r0, A.W);
    const int ng = nb * A.G;
    const int TG = A.TG;
    const int64_t gbase = ((int64_t)bs * A.Hkv + kvh) * A.max_chunks * A.G;
    const bf16_t* gk = reinterpret_cast<const bf16_t*>(A.index + A.L.gk) + gbase * kD;
    const float* gln = reinterpret_cast<const float*>(A.index + A.L.gln) + gbase;
    const float* gkn = reinterpret_cast<const float*>(A.index + A.L.gkn) + gbase;
    auto qrow = [&](int n) {  // column n -> its query row (clamped into the tile)
        const int rl = min(n / HG, nrows - 1);
        return A.q + (((int64_t)b * A.nq + r0 + rl) * A.Hq + hq0 + n % HG) * kD;
    };
    // column n -> (list slot of this split), -1 for columns past the last row
    auto list_at = [&](int n) -> int64_t {
        const int rl = n / HG;
        if (rl >= nrows) return -1;
        const int64_t col = ((int64_t)b * A.nq + r0 + rl) * A.Hq + hq0 + n % HG;
        return col * A.nsplit + split;
    };

    // Q^T operands of this lane's two columns, |q| per column
    bf16x8_t qb[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int n = 16 * (2 * w + cb) + (l & 15);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qb[cb][kk] = *reinterpret_cast<const bf16x8_t*>(qrow(n) + 32 * kk + 8 * (l >> 4));
    }
    if (tid < kFlashRowHeads) {
        const bf16_t* qr = qrow(tid);
        float ss = 0.0f;
        for (int c = 0; c < 16; ++c) {
            float f[8];
            Elt<bf16_t>::unpack(*reinterpret_cast<const uint4*>(qr + 8 * c), f);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
        }
        s.qn[tid] = sqrtf(ss) * 1.0001f;
        s.cnt[tid] = 0;
    }
    __syncthreads();
    const float qn[2] = {s.qn[16 * (2 * w) + (l & 15)], s.qn[16 * (2 * w + 1) + (l & 15)]};

    // MFMA scores S^T of key block kb (16 keys) of one staged tile for this lane's two
    // columns; ktb: the tile's row l % 16, lo_: l % 16 (key row 16 kb + l % 16 holds
    // chunk 4 kk + l / 16 at (4 kk + l / 16) ^ (l % 16))
    auto block_scores = [&](f32x4_t* S, const bf16_t* ktb, int lo_, int kb) {
        S[0] = {0.0f, 0.0f, 0.0f, 0.0f};
        S[1] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ktb + 16 * kb * kD + 8 * ((4 * kk + (l >> 4)) ^ lo_));
            S[0] = mfma16(a, qb[0][kk], S[0]);
            S[1] = mfma16(a, qb[1][kk], S[1]);
        }
    };
    // This split's centroid tiles [t0, t1) of 64 groups stream through two LDS buffers:
    // the loads of tile t+1 (keys, ln n and norm bounds, all straight to LDS) are in
    // flight while tile t is used.  Each wave waits for its own older loads (vmcnt: the
    // 4, or 6 in wave 0, instructions of the newer tile may stay outstanding), then a
    // barrier publishes.
    const int ntile = (ng + kFlashKeys - 1) / kFlashKeys;
    const int t0 = (int)((int64_t)ntile * split / A.nsplit);
    const int t1 = (int)((int64_t)ntile * (split + 1) / A.nsplit);
    auto issue = [&](int t) {
        const int buf = (t - t0) & 1, g0 = t * kFlashKeys, nk = min(kFlashKeys, ng - g0);
        stage_rows_swizzled(s.kt[buf], gk + (int64_t)g0 * kD, nk);
        if (w == 0) {
            const int g = g0 + min(l, nk - 1);
            __builtin_amdgcn_global_load_lds(gln + g, &s.gln_t[buf][0], 4, 0, 0);
            __builtin_amdgcn_global_load_lds(gkn + g, &s.gkn_t[buf][0], 4, 0, 0);
        }
    };
    auto await_tile = [&](int t) {
        if (t + 1 < t1) {
            if (w == 0) __builtin_amdgcn_s_waitcnt(0xF76);  // vmcnt <= 6
            else __builtin_amdgcn_s_waitcnt(0xF74);         // vmcnt <= 4
        } else {
            __builtin_amdgcn_s_waitcnt(0);
        }
        lds_barrier();
    };
    // sweep over the split's tiles; body(t, buf, nk, kb, S) sees the MFMA scores of key
    // block kb.  WT: the scores of the whole tile first (more MFMAs in flight per wave,
    // for launches of few waves per SIMD), else one block at a time (8 registers of
    // scores live instead of 32: four waves per SIMD)
    auto sweep = [&](auto&& body) {
        if (t0 < t1) issue(t0);
        for (int t = t0; t < t1; ++t) {
            if (t + 1 < t1) issue(t + 1);
            await_tile(t);
            const int buf = (t - t0) & 1;
            const int nk = min(kFlashKeys, ng - t * kFlashKeys);
            // LDS addresses formed from a lane value the compiler cannot see through, once
            // per tile, so none is hoisted out of the loop into a register of its own
            int lo_ = l & 15;
            asm volatile("" : "+v"(lo_));
            const bf16_t* ktb = &s.kt[buf][0][0] + lo_ * kD;
            if constexpr (WT) {
                f32x4_t S[4][2];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) block_scores(S[kb], ktb, lo_, kb);
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) body(t, buf, nk, kb, S[kb]);
            } else {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    f32x4_t S[2];
                    block_scores(S, ktb, lo_, kb);
                    body(t, buf, nk, kb, S);
                }
            }
            lds_barrier();  // the buffer is free for tile t + 2
        }
    };

    // pass A: per column, large lower bounds S - E.  Each lane keeps the R largest of its
    // 4-key blocks' maxima (one insertion per block instead of one per key: the values
    // are still lower bounds of distinct groups, so the TG-th largest of the four lanes'
    // lists is still at or below the split's TG-th largest lower bound), in lists kept
    // sorted by a branch-free insertion.
    float lst[2][R];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int e = 0; e < R; ++e) lst[cb][e] = -INFINITY;
    float pinf = INFINITY;  // +inf the compiler cannot see (insert_desc's head med3)
    asm volatile("" : "+v"(pinf));
    sweep([&](int, int buf, int nk, int kb, f32x4_t* S) {
            // ln n and norm bounds of this lane's four keys (every one of the 64 slots is
            // staged, so the reads need no branch)
            const int k4 = 16 * kb + 4 * (l >> 4);
            const float4 gl4 = *reinterpret_cast<const float4*>(&s.gln_t[buf][k4]);
            const float4 gn4 = *reinterpret_cast<const float4*>(&s.gkn_t[buf][k4]);
            const float glr[4] = {gl4.x, gl4.y, gl4.z, gl4.w}, gnr[4] = {gn4.x, gn4.y, gn4.z, gn4.w};
            float bm[2] = {-INFINITY, -INFINITY};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool valid = (k4 + r < nk) & (glr[r] != -INFINITY);
                const float gn = gnr[r];
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    bm[cb] = fmaxf(bm[cb], valid ? S[cb][r] - kErrC * qn[cb] * gn : -INFINITY);
            }
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) insert_desc(lst[cb], bm[cb], pinf);
    });
    // merge the four lanes of each column: the TG largest with multiplicity, descending;
    // the local threshold is the TG-th (-inf when the split has fewer valid groups)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int n = 16 * (2 * w + cb) + (l & 15);
        const int64_t at = list_at(n);
        float* top = (at >= 0 && (l >> 4) == 0) ? A.ltop + at * kMaxTG : nullptr;
        int taken = 0;
        float T = -INFINITY;
        for (int round = 0; round < TG && taken < TG; ++round) {
            float h = lst[cb][0];
            float m = fmaxf(h, __shfl_xor(h, 16, 64));
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            const int mine = (h == m && m != -INFINITY) ? 1 : 0;
            int c = mine + __shfl_xor(mine, 16, 64);
            c += __shfl_xor(c, 32, 64);
            if (m == -INFINITY) break;  // uniform over the column's four lanes
            const int upto = min(taken + c, TG);
            if (top)
                for (int e = taken; e < upto; ++e) top[e] = m;
            taken = upto;
            if (taken >= TG) T = m;
            if (mine) {
#pragma unroll
                for (int e = 0; e < R - 1; ++e) lst[cb][e] = lst[cb][e + 1];
                lst[cb][R - 1] = -INFINITY;
            }
        }
        if (top)
            for (int e = taken; e < TG; ++e) top[e] = -INFINITY;
        if ((l >> 4) == 0) s.T[n] = T;
    }
    __syncthreads();

    // pass B: this split's candidates S + E >= T
    const float T2[2] = {s.T[16 * (2 * w) + (l & 15)], s.T[16 * (2 * w + 1) + (l & 15)]};
    const int64_t lat[2] = {list_at(16 * (2 * w) + (l & 15)), list_at(16 * (2 * w + 1) + (l & 15))};
    sweep([&](int t, int buf, int nk, int kb, f32x4_t* S) {
        const int g0 = t * kFlashKeys;
        // this lane's candidates of key block kb as bit masks (bit r)
        uint32_t m[2] = {0u, 0u};
        const int k4 = 16 * kb + 4 * (l >> 4);
        const float4 gl4 = *reinterpret_cast<const float4*>(&s.gln_t[buf][k4]);
        const float4 gn4 = *reinterpret_cast<const float4*>(&s.gkn_t[buf][k4]);
        const float glr[4] = {gl4.x, gl4.y, gl4.z, gl4.w}, gnr[4] = {gn4.x, gn4.y, gn4.z, gn4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool valid = (k4 + r < nk) & (glr[r] != -INFINITY);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const float ub = S[cb][r] + kErrC * qn[cb] * gnr[r];
                m[cb] |= (valid & (ub >= T2[cb])) ? (1u << r) : 0u;
            }
        }
        // one LDS atomic per lane, column and key block with candidates, then the entries
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            if (m[cb] == 0u) continue;
            const int n = 16 * (2 * w + cb) + (l & 15);
            int at = atomicAdd(&s.cnt[n], __popc(m[cb]));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if ((m[cb] >> r) & 1u) {
                    if (at < kSplitCap && lat[cb] >= 0) {
                        const float ub = S[cb][r] + kErrC * qn[cb] * gnr[r];
                        A.lent[lat[cb] * kSplitCap + at] = make_uint2((uint32_t)(g0 + k4 + r), __float_as_uint(ub));
                    }
                    ++at;
                }
            }
        }
    });
    if (tid < kFlashRowHeads) {
        const int64_t at = list_at(tid);
        if (at >= 0) A.lcnt[at] = s.cnt[tid];
    }
}

constexpr int kSelCols = 64;  // (row, head) columns per select workgroup: half a column tile

template <int NC>
struct SelSmem {
    float T[NC];
    int cnt[NC];
    // per-column rows padded to an odd number of words: lanes that read one column each
    // hit distinct LDS banks
    int32_t cg[NC][kCandCap + 1];  // candidates: group id, upper bound of the canonical
    float cub[NC][kCandCap + 1];   // score (then the score itself where computed),
    float clb[NC][kCandCap + 1];   // lower bound, class (0 surely not opened, 1
    uint8_t cls[NC][kCandCap + 4]; // needs the chain, 2 surely opened)
    float qn[NC];                  // |q| per column, rounded up
    int32_t sel[NC][kMaxTG + 1];   // rank order
    int nsel[NC];
    uint64_t red[4];
    int any_overflow;
};

// Selection of NC (row, head) columns -- columns c0 .. c0 + NC - 1 of a 128-column tile
// -- from the candidate lists of the sweeps: global threshold, candidates, exact top TG
// under the canonical chain, then page ranking of every opened group.
// TGM: opened groups per column at most (8 or kMaxTG): the sorting networks are sized by it.
template <int HG, int NC, int TGM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void prefill_select_kernel(SelArgs A) {
    __shared__ SelSmem<NC> s;
    constexpr int QT = kFlashRowHeads / HG;
    const SelSlot slot = sel_slot(A.Hkv, kFlashRowHeads / NC);  // split field: the column group
    const int c0 = slot.split * NC;
    const int tile = slot.tile, kvh = slot.kvh, b = blockIdx.z, bs = A.seq + b;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int r0 = tile * QT;
    const int nrows = min(QT, A.nq - r0);
    const int hq0 = kvh * HG;
    const int nb = nbuilt_prefill(A.pos0 + r0, A.W);
    const int ng = nb * A.G;
    const int TG = A.TG;
    const int TPW = A.TP > 0 ? A.TP : 1;
    const int64_t gbase = ((int64_t)bs * A.Hkv + kvh) * A.max_chunks * A.G;
    const bf16_t* gk = reinterpret_cast<const bf16_t*>(A.index + A.L.gk) + gbase * kD;
    const float* gln = reinterpret_cast<const float*>(A.index + A.L.gln) + gbase;
    auto qrow = [&](int n) {  // column n -> its query row (clamped into the tile)
        const int rl = min((c0 + n) / HG, nrows - 1);
        return A.q + (((int64_t)b * A.nq + r0 + rl) * A.Hq + hq0 + (c0 + n) % HG) * kD;
    };
    auto col_of = [&](int n) { return ((int64_t)b * A.nq + r0 + (c0 + n) / HG) * A.Hq + hq0 + (c0 + n) % HG; };

    // global threshold per column: the TG-th largest of the splits' top lists (they hold
    // the TG largest lower bounds of every split, hence those of all groups)
    if (tid < NC) {
        const int n = tid;
        float T = -INFINITY;
        int over = 0;
        if ((c0 + n) / HG < nrows) {
            const int64_t c0 = col_of(n) * A.nsplit;
            float top[TGM];
#pragma unroll
            for (int e = 0; e < TGM; ++e) top[e] = -INFINITY;
            for (int sp = 0; sp < A.nsplit; ++sp) {
                over |= A.lcnt[c0 + sp] > kSplitCap;
                const float4* src = reinterpret_cast<const float4*>(A.ltop + (c0 + sp) * kMaxTG);
                float v[TGM];
#pragma unroll
                for (int i = 0; i < TGM / 4; ++i) {
                    const float4 f = 4 * i < TG ? src[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
                    v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
                }
#pragma unroll
                for (int i = 0; i < TGM; ++i) {
                    const float x = i < TG ? v[i] : -INFINITY;
                    if (x > top[TGM - 1]) insert_desc(top, x);
                }
            }
#pragma unroll
            for (int e = 0; e < TGM; ++e)
                if (e == TG - 1) T = top[e];
        }
        s.T[n] = T;
        s.cnt[n] = over ? kCandCap + 1 : 0;  // an overflowed split forces the exhaustive path
        // |q| rounded up, computed as the sweep computed it
        const bf16_t* qr = qrow(n);
        float ss = 0.0f;
        for (int c = 0; c < 16; ++c) {
            float f[8];
            Elt<bf16_t>::unpack(*reinterpret_cast<const uint4*>(qr + 8 * c), f);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(f[e], f[e], ss);
        }
        s.qn[n] = sqrtf(ss) * 1.0001f;
    }
    if (tid == 0) s.any_overflow = 0;
    __syncthreads();
    // candidates: listed groups with upper bound >= the global threshold (two threads per
    // column, alternate splits), with lower bounds ub - 2E (E = kErrC |q| |kbar| as the
    // sweep computed it, from the stored norm bound)
    const float* gkn = reinterpret_cast<const float*>(A.index + A.L.gkn) + gbase;
    {
        const int n = tid & (NC - 1);
        if ((c0 + n) / HG < nrows) {
            const int64_t c0 = col_of(n) * A.nsplit;
            const float T = s.T[n];
            for (int sp = tid / NC; sp < A.nsplit; sp += kThreads / NC) {
                const int c = min(A.lcnt[c0 + sp], kSplitCap);
                const uint4* src = reinterpret_cast<const uint4*>(A.lent + (c0 + sp) * kSplitCap);
                uint4 e[kSplitCap / 2];
#pragma unroll
                for (int i = 0; i < kSplitCap / 2; ++i)
                    if (2 * i < c) e[i] = src[i];
                const float e2 = 2.0f * kErrC * s.qn[n];
#pragma unroll
                for (int i = 0; i < kSplitCap / 2; ++i) {
                    if (2 * i < c && __uint_as_float(e[i].y) >= T) {
                        const int at = atomicAdd(&s.cnt[n], 1);
                        if (at < kCandCap) {
                            const float ub = __uint_as_float(e[i].y);
                            s.cg[n][at] = (int32_t)e[i].x;
                            s.cub[n][at] = ub;
                            s.clb[n][at] = ub - e2 * gkn[e[i].x];
                        }
                    }
                    if (2 * i + 1 < c && __uint_as_float(e[i].w) >= T) {
                        const int at = atomicAdd(&s.cnt[n], 1);
                        if (at < kCandCap) {
                            const float ub = __uint_as_float(e[i].w);
                            s.cg[n][at] = (int32_t)e[i].z;
                            s.cub[n][at] = ub;
                            s.clb[n][at] = ub - e2 * gkn[e[i].z];
                        }
                    }
                }
            }
        }
    }
    __syncthreads();

    // certification: a candidate is surely opened when fewer than TG others can reach its
    // lower bound (the TG-th largest upper bound of the others is below it), surely not
    // when TG others are above its upper bound (the TG-th largest lower bound is above
    // it); only the rest need the canonical chain (all of them when the rank order is an
    // output).  Needs the TG and TG+1 largest upper bounds and the TG largest lower bounds.
    if (tid < NC) {
        const int n = tid, c = s.cnt[n];
        if (c <= kCandCap) {
            float tu[TGM + 1], tl[TGM];
#pragma unroll
            for (int e = 0; e <= TGM; ++e) tu[e] = -INFINITY;
#pragma unroll
            for (int e = 0; e < TGM; ++e) tl[e] = -INFINITY;
            for (int at = 0; at < c; ++at) {
                insert_desc(tu, s.cub[n][at]);
                insert_desc(tl, s.clb[n][at]);
            }
            float uT = -INFINITY, uT1 = -INFINITY, lT = -INFINITY;  // TG-th, TG+1-th largest ub; TG-th lb
#pragma unroll
            for (int e = 0; e <= TGM; ++e) {
                if (e == TG - 1) { uT = tu[e]; lT = e < TGM ? tl[e] : -INFINITY; }
                if (e == TG) uT1 = tu[e];
            }
            for (int at = 0; at < c; ++at) {
                const float lb = s.clb[n][at], ub = s.cub[n][at];
                const float others = ub >= uT ? uT1 : uT;  // TG-th largest ub of the others
                s.cls[n][at] = (!A.sel_groups && lb > others) ? 2 : (lT > ub ? 0 : 1);
            }
        }
    }
    __syncthreads();
    // canonical chains for the candidates that need them (the score replaces the bound).
    // A column past kCandCap takes the exhaustive path below and skips this: its classes
    // were never set, and when a split's list overflowed, not even its candidate slots
    // (their group ids would be whatever LDS held).
    for (int x = tid; x < NC * kCandCap; x += kThreads) {
        const int n = x / kCandCap, at = x % kCandCap;
        const int c = s.cnt[n];
        if (c <= kCandCap && at < c && s.cls[n][at] == 1)
            s.cub[n][at] = canonical_dot_bf16(qrow(n), gk + (int64_t)s.cg[n][at] * kD);
    }
    __syncthreads();
    // exact top-TG per column among its candidates (columns that overflowed: below)
    if (tid < NC) {
        const int n = tid, c = s.cnt[n];
        if (c > kCandCap) {
            atomicOr(&s.any_overflow, 1);
            s.nsel[n] = -1;
        } else {
            uint64_t top[TGM];
#pragma unroll
            for (int e = 0; e < TGM; ++e) top[e] = 0;
            for (int at = 0; at < c; ++at) {
                // ranking key: surely opened above every score (ties to the lower id),
                // surely not 0 (never opened), else the canonical score
                const uint32_t id = (uint32_t)s.cg[n][at];
                const int cl = s.cls[n][at];
                uint64_t x = cl == 2 ? ((0xffffffffull << 32) | (0xffffffffu - id))
                                     : (cl == 0 ? 0ull : rank_key(s.cub[n][at], id));
#pragma unroll
                for (int e = 0; e < TGM; ++e) {
                    const uint64_t hi = top[e] > x ? top[e] : x, lo = top[e] > x ? x : top[e];
                    top[e] = hi;
                    x = lo;
                }
            }
            int k = 0;  // surely-out candidates (key 0) are never opened
#pragma unroll
            for (int e = 0; e < TGM; ++e) k += (e < TG && top[e] != 0) ? 1 : 0;
#pragma unroll
            for (int e = 0; e < TGM; ++e)
                if (e < TG) s.sel[n][e] = e < k ? (int)key_id(top[e]) : -1;
            s.nsel[n] = k;
        }
    }
    __syncthreads();
    // exhaustive path for columns with more candidates than kept: canonical scores of
    // every eligible group, workgroup-wide top-TG
    if (s.any_overflow) {
        for (int n = 0; n < NC; ++n) {
            if (s.nsel[n] >= 0) continue;  // uniform: read from LDS after a barrier
            uint64_t top[TGM];
#pragma unroll
            for (int e = 0; e < TGM; ++e) top[e] = 0;
            for (int g = tid; g < ng; g += kThreads) {
                if (gln[g] == -INFINITY) continue;
                uint64_t x = rank_key(canonical_dot_bf16(qrow(n), gk + (int64_t)g * kD), (uint32_t)g);
#pragma unroll
                for (int e = 0; e < TGM; ++e) {
                    const uint64_t hi = top[e] > x ? top[e] : x, lo = top[e] > x ? x : top[e];
                    top[e] = hi;
                    x = lo;
                }
            }
            int k = 0;
            for (int round = 0; round < TG; ++round) {
                const uint64_t wm = wave_max_u64(top[0]);
                if (l == 0) s.red[w] = wm;
                __syncthreads();
                uint64_t m = s.red[0];
                for (int x = 1; x < 4; ++x) m = s.red[x] > m ? s.red[x] : m;
                __syncthreads();
                if (m == 0) break;
                if (tid == 0) s.sel[n][round] = (int)key_id(m);
                if (top[0] == m) {
#pragma unroll
                    for (int e = 0; e < TGM - 1; ++e) top[e] = top[e + 1];
                    top[TGM - 1] = 0;
                }
                ++k;
            }
            if (tid == 0) {
                for (int e = k; e < TG; ++e) s.sel[n][e] = -1;
                s.nsel[n] = k;
            }
            __syncthreads();
        }
    }

    // outputs: opened groups (rank order and ascending), then the pages of each
    for (int x = tid; x < NC * TG; x += kThreads) {
        const int n = x / TG, t = x % TG;
        const int rl = (c0 + n) / HG;
        if (rl >= nrows) continue;
        const int64_t rh = ((int64_t)b * A.nq + r0 + rl) * A.Hq + hq0 + (c0 + n) % HG;
        if (A.sel_groups) A.sel_groups[rh * TG + t] = s.sel[n][t];
        // ascending copy: the t-th smallest id among the selected
        const int gt = s.sel[n][t];
        int pos = 0;
        for (int e = 0; e < s.nsel[n]; ++e) pos += s.sel[n][e] < gt;
        if (gt >= 0) A.selg[rh * TG + pos] = gt;
        if (t >= s.nsel[n]) A.selg[rh * TG + t] = -1;
    }
    const int16_t* meta_u = reinterpret_cast<const int16_t*>(A.index + A.L.meta) +
                            ((int64_t)bs * A.Hkv + kvh) * A.max_chunks * A.L.meta_stride;
    const bf16_t* pk_u = reinterpret_cast<const bf16_t*>(A.index + A.L.pk) +
                         ((int64_t)bs * A.Hkv + kvh) * A.max_chunks * A.L.page_slots * kD;
    for (int x = tid; x < NC * TG; x += kThreads) {
        const int n = x / TG, t = x % TG;
        const int rl = (c0 + n) / HG;
        if (rl >= nrows) continue;
        const int64_t rh = ((int64_t)b * A.nq + r0 + rl) * A.Hq + hq0 + (c0 + n) % HG;
        PairRec R;
        R.gid = s.sel[n][t];
        R.ps0 = R.npg = 0;
        R.open = 0;
        int slot_rank[kPage];
#pragma unroll
        for (int e = 0; e < kPage; ++e) { R.r[e] = 0.0f; slot_rank[e] = -1; }
        if (R.gid >= 0) {
            const int c = R.gid / A.G, j = R.gid % A.G;
            const int16_t* gpg = meta_u + (int64_t)c * A.L.meta_stride;
            const int ps0 = gpg[j], npg = gpg[j + 1] - ps0;
            R.ps0 = (int16_t)ps0;
            R.npg = (int16_t)npg;
            if (A.TP == 0 || (npg <= A.TP && !A.sel_pages)) {
                // every page opened: no ranking, and no unopened page needs a logit
                R.open = npg >= 32 ? 0xffffffffu : ((1u << npg) - 1u);
            } else {
                uint64_t key[kPage];  // every index below is static: the record stays in registers
#pragma unroll
                for (int e = 0; e < kPage; ++e) {
                    key[e] = 0;
                    if (e < npg) {
                        R.r[e] = canonical_dot_bf16(qrow(n), pk_u + ((int64_t)c * A.L.page_slots + ps0 + e) * kD);
                        key[e] = rank_key(R.r[e], (uint32_t)e);
                    }
                }
                const int nopen = min(npg, A.TP);
#pragma unroll
                for (int k = 0; k < kPage; ++k) {
                    if (k < nopen) {
                        // largest remaining key (register-resident: static indices only)
                        uint64_t bk = 0;
                        int best = 0;
#pragma unroll
                        for (int e = 0; e < kPage; ++e)
                            if (key[e] > bk) { bk = key[e]; best = e; }
#pragma unroll
                        for (int e = 0; e < kPage; ++e)
                            if (e == best) key[e] = 0;
                        slot_rank[k] = best;
                        R.open |= 1u << best;
                    }
                }
            }
        }
        // records go in ascending group order (the order of selg), so later steps read
        // the compact selg array to find a slot's group
        int pos = t;
        if (R.gid >= 0) {
            pos = 0;
            for (int e = 0; e < s.nsel[n]; ++e) pos += s.sel[n][e] < R.gid;
        }
        A.rec[rh * TG + pos] = R;
        if (R.gid < 0) A.part_pg[(rh * TG + pos) * kPartStride + kD] = -INFINITY;  // no pages kernel pair
        if (A.sel_pages) {
#pragma unroll
            for (int k = 0; k < kPage; ++k)
                if (k < TPW)
                    A.sel_pages[(rh * TG + t) * TPW + k] =
                        (A.TP > 0 && R.gid >= 0 && slot_rank[k] >= 0) ? R.ps0 + slot_rank[k] : -1;
        }
    }
}
// ---------------------------------------------------------------------------- bucket

// A unit is (sequence, KV head, 256-row query chunk of the launch); its pairs are
// (row, head, slot) with pair index (row_in_chunk * HG + head) * TG + slot.
constexpr int kMaxBucketGroups = 16384;  // summarised groups per KV head a prefill supports
constexpr int kBucketThreads = 1024;     // threads of a bucket workgroup

struct PagesArgs {
    const bf16_t* k;
    const bf16_t* v;
    int64_t sb, st, sh;
    const int32_t* btab;  // paged view: block table [batch][maxb], else null
    int bshift, maxb;
    const bf16_t* q;
    int seq;                // sequence of grid slice z = 0 (index and cache)
    int nq, pos0, Hq, Hkv;
    float scale;
    const char* index;
    lod_index_layout_t L;
    int max_chunks, G, W, TG;
    int drop;               // 1: no coarse remainder (unopened pages add nothing)
    int q4;                 // 1: opened rows decoded from the index's 4-bit codes
    int tp;                 // pages opened per opened group (0: two-tier, every page)
    const PairRec* rec;     // [B][nq][Hq][TG], slot t holds the group selg[t]
    const int32_t* selg;    // [B][nq][Hq][TG] opened groups, ascending (-1 padding)
    int2* plist;            // [units][kChunk * HG * TG] (pair index, group) sorted by group
    int32_t* poff;          // [units][2]: number of pairs with a group, (unused)
    float* part_fl;         // [nsplit][B][nq][Hq] flash partial states
    int nsplit;
    int64_t split_stride;
    float* part_pg;         // [B][nq][Hq][TG] page partial states
    float* out;             // [B][nq][Hq][d]
    int units_per_seq_kv;   // query chunks in the launch
};

// Counting sort of one unit's (query chunk qc, KV head kvh, sequence b) pairs by opened
// group, by NT threads.  PER: pair slots per thread, at least kChunk * HG * TG / NT.
// cnt: kMaxBucketGroups + 64 counters (+ 64 spares: slots with no group, or past the last
// pair, count into the spare of their lane, so every slot takes its atomic without a
// branch); wsum: NT / 64 words.  STAGE (up to 16 slots per thread, 16384 pairs): the
// sorted list is assembled in stage[NT * 16] (pair index and group in 14 bits each) and
// written out in order, so the global stores are coalesced instead of scattered one pair
// at a time.
template <int HG, int PER, int NT, bool STAGE>
__device__ __forceinline__ void bucket_body(const PagesArgs& A, int qc, int kvh, int b, int* cnt, uint32_t* stage,
                                            int* wsum) {
    const int tid = threadIdx.x;
    const int r0 = qc * kChunk;
    const int nrows = min(kChunk, A.nq - r0);
    const int nb = nbuilt_prefill(A.pos0 + r0, A.W);
    const int ng = nb * A.G;
    const int npairs = nrows * HG * A.TG;
    const int64_t unit = ((int64_t)b * A.Hkv + kvh) * A.units_per_seq_kv + qc;
    int2* list = A.plist + unit * (kChunk * HG * A.TG);
    for (int g = tid; g < ng; g += NT) cnt[g] = 0;
    const int spare = kMaxBucketGroups + (tid & 63);
    // the group id of every pair this thread owns (pairs tid, tid + NT, ...), loaded
    // together and kept for both passes.  Pair x = rl * HG * TG + e (e = head * TG + slot)
    // sits at selg row r0 + rl, entry kvh * HG * TG + e; (rl, e) advances by the
    // division of NT by HG * TG with one carry, so the loop divides nothing.
    int gid[PER];
    {
        const int per_row = HG * A.TG, rs = A.Hq * A.TG;  // pairs of a unit row; selg row stride
        const int de = NT % per_row, doff = NT / per_row * rs + de;
        int e = tid % per_row, off = tid / per_row * rs + e;
        const int32_t* sg = A.selg + ((int64_t)b * A.nq + r0) * rs + kvh * per_row;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            gid[u] = tid + u * NT < npairs ? sg[off] : -1;
            off += doff;
            e += de;
            if (e >= per_row) { e -= per_row; off += rs - per_row; }
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) atomicAdd(&cnt[gid[u] >= 0 ? gid[u] : spare], 1);
    __syncthreads();
    // exclusive scan of the counts: contiguous ranges per thread, then the range sums by
    // wave prefix sums and the waves' totals
    const int per = (ng + NT - 1) / NT;
    const int g0 = tid * per, g1 = min(ng, g0 + per);
    int sum = 0;
    for (int g = g0; g < g1; ++g) sum += cnt[g];
    const int lane = tid & 63, wv = tid >> 6;
    int incl = sum;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
        const int o = __shfl_up(incl, sh, 64);
        if (lane >= sh) incl += o;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int x = 0; x < NT / 64; ++x) {
        before += x < wv ? wsum[x] : 0;
        total += wsum[x];
    }
    if (tid == 0) A.poff[unit * 2] = total;
    int acc = before + incl - sum;
    for (int g = g0; g < g1; ++g) { const int v = cnt[g]; cnt[g] = acc; acc += v; }
    __syncthreads();
    // every slot's LDS atomic first, then the stores (one wait, not one per pair)
    int at[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) at[u] = atomicAdd(&cnt[gid[u] >= 0 ? gid[u] : spare], 1);
    if constexpr (STAGE) {
#pragma unroll
        for (int u = 0; u < PER; ++u)
            if (gid[u] >= 0) stage[at[u]] = (uint32_t)(tid + u * NT) | ((uint32_t)gid[u] << 14);
        __syncthreads();
        for (int x = tid; x < total; x += NT) {
            const uint32_t v = stage[x];
            list[x] = make_int2((int)(v & 0x3fffu), (int)(v >> 14));
        }
    } else {
#pragma unroll
        for (int u = 0; u < PER; ++u)
            if (gid[u] >= 0) list[at[u]] = make_int2(tid + u * NT, gid[u]);
    }
}

// PER: pair slots per thread, at least kChunk * HG * TG / kBucketThreads.
template <int HG, int PER>
__global__ __launch_bounds__(kBucketThreads) void prefill_bucket_kernel(PagesArgs A) {
    __shared__ int cnt[kMaxBucketGroups + 64];
    constexpr bool kStage = PER <= 16;
    __shared__ uint32_t stage[kStage ? kBucketThreads * 16 : 1];
    __shared__ int wsum[kBucketThreads / 64];
    bucket_body<HG, PER, kBucketThreads, kStage>(A, blockIdx.x, blockIdx.y, blockIdx.z, cnt, stage, wsum);
}

// The flash kernel and the bucket sort in one launch: both need only the selection, so
// the bucket workgroups (after the nflash flash workgroups, one per query chunk and KV
// head) take the CUs that the first flash workgroups to end leave, beside the flash
// tail, instead of running as a launch of their own between the flash kernel and the
// group kernel, where eight workgroups held the whole GPU for about 10 us per call.  The
// bucket side sorts with the flash kernel's 512 threads and without staging (its LDS is
// the flash kernel's, whose 75 KB would not also hold the stage).
template <int HG>
union FlashBucketSmem {
    FlashSmem<HG> f;
    struct {
        int cnt[kMaxBucketGroups + 64];
        int wsum[kFlashThreads / 64];
    } k;
};

template <int HG, bool PAGED, int PER>
__global__ __launch_bounds__(kFlashThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void prefill_flash_bucket_kernel(FlashArgs F, PagesArgs P, int nflash, int nunits_q) {
    __shared__ FlashBucketSmem<HG> u;
    const int bx = blockIdx.x;
    if (bx >= nflash) {  // uniform in the workgroup
        const int x = bx - nflash;
        bucket_body<HG, PER, kFlashThreads, false>(P, x % nunits_q, x / nunits_q, blockIdx.z, u.k.cnt, nullptr,
                                                   u.k.wsum);
        return;
    }
    flash_body<HG, PAGED>(F, u.f, bx);
}

// ---------------------------------------------------------------------------- pages

constexpr int kPairsPerWG = 16;  // one (row, head, slot) pair per 16-lane subgroup
constexpr int kPagesMeta = 320;  // int16 entries of a chunk's meta row held in LDS (>= meta_stride)

// One workgroup per 16 consecutive pairs of a unit's group-sorted list; each 16-lane
// subgroup runs one pair: exact rows of its opened pages and the mean terms of the
// unopened pages of its group, one online softmax, written as the pair's partial state.
// Pairs of the same group run side by side, so their rows come from the same cache lines.
// A pair's loads form three dependent steps: its list entry (pair and group); the query,
// its record and the whole meta row of the group's chunk (to LDS); then the rows of the
// opened pages (batches of 8, kept packed) with the unopened pages' means.
// Q4: the opened rows are decoded from the index's 4-bit codes (fma(scale, code, group
// mean)), so no cache row is read.
template <int HG, bool PAGED, bool Q4>
__global__ __launch_bounds__(kThreads) void prefill_pages_kernel(PagesArgs A) {
    __shared__ alignas(16) int16_t mrow[kPairsPerWG][kPagesMeta];
    const int blk = blockIdx.x, unit_local = blockIdx.y;
    const int qc = unit_local % A.units_per_seq_kv;
    const int kvh = (unit_local / A.units_per_seq_kv) % A.Hkv;
    const int b = unit_local / (A.units_per_seq_kv * A.Hkv);
    const int tid = threadIdx.x, l16 = tid & 15, sg = tid >> 4;
    const int64_t unit = unit_local;
    const int npairs = A.poff[unit * 2];
    const int r0 = qc * kChunk;
    const int PS = A.L.page_slots;
    const int2* list = A.plist + unit * (kChunk * HG * A.TG);
    const int bs = A.seq + b;
    const int64_t ubase = ((int64_t)bs * A.Hkv + kvh) * A.max_chunks;
    const int16_t* meta_u = reinterpret_cast<const int16_t*>(A.index + A.L.meta) + ubase * A.L.meta_stride;
    const bf16_t* pv_u = reinterpret_cast<const bf16_t*>(A.index + A.L.pv) + ubase * PS * kD;
    const float* pln_u = reinterpret_cast<const float*>(A.index + A.L.pln) + ubase * PS;
    // head kvh of sequence bs; the row of position x adds kv_pos(A, bs, x)
    const bf16_t* kc = A.k + kvh * A.sh + kv_seq<PAGED>(A, bs);
    const bf16_t* vc = A.v + kvh * A.sh + kv_seq<PAGED>(A, bs);

    const int x = blk * kPairsPerWG + sg;
    if (x >= npairs) return;  // uniform in the subgroup
    const int seg0 = (tid & 63) & ~15;
    const int2 le = list[x];
    const int pi = le.x, gid = le.y;
    const int t = pi % A.TG, h = (pi / A.TG) % HG, rl = pi / (A.TG * HG);
    const int64_t rh = ((int64_t)b * A.nq + r0 + rl) * A.Hq + kvh * HG + h;
    const int c = gid / A.G, j = gid % A.G;
    // step 2: query, record, meta row
    float q8[8];
    load8<bf16_t>(A.q + rh * kD, l16, q8);
    const PairRec* R = A.rec + rh * A.TG + t;
    const uint32_t open = R->open;
    const float rl16 = R->r[l16];  // lane e: score of page e
    {
        // 16-byte pieces l16, l16 + 16, l16 + 32 of the row (a meta row has 36 to 40)
        const int ms16 = A.L.meta_stride / 8;
        const uint4* src = reinterpret_cast<const uint4*>(meta_u + (int64_t)c * A.L.meta_stride);
        const uint4 m0 = src[l16], m1 = src[l16 + 16], m2 = src[min(l16 + 32, ms16 - 1)];
        *reinterpret_cast<uint4*>(&mrow[sg][8 * l16]) = m0;
        *reinterpret_cast<uint4*>(&mrow[sg][8 * (l16 + 16)]) = m1;
        if (l16 + 32 < ms16) *reinterpret_cast<uint4*>(&mrow[sg][8 * (l16 + 32)]) = m2;
    }
    wave_sync_lds();
    const int16_t* gpg = &mrow[sg][0];
    const int16_t* pst = gpg + (A.G + 1);
    const int16_t* perm = pst + (PS + 1);
    const int ps0 = gpg[j], npg = gpg[j + 1] - ps0;
    const uint32_t pmask = npg >= 32 ? 0xffffffffu : (1u << npg) - 1u;
    const uint32_t opened = open & pmask, closed = A.drop ? 0u : ~open & pmask;
    // step 3: ln n of the unopened pages, the opened rows; then the unopened pages' means
    // (rare: a group's pages beyond the top ones)
    const float pln16 = (closed >> l16) & 1u ? pln_u[(int64_t)c * PS + ps0 + l16] : 0.0f;  // lane e: page e
    // opened rows in page order: row u of the pair is member u - start(e) of opened page e
    int nrow = 0;
    for (uint32_t m = opened; m; m &= m - 1) {
        const int e = __builtin_ctz(m);
        nrow += pst[ps0 + e + 1] - pst[ps0 + e];
    }
    auto row_pos = [&](int u) {  // position of opened row u (u < nrow)
        int base = 0;
        for (uint32_t m = opened; m; m &= m - 1) {
            const int e = __builtin_ctz(m);
            const int x0 = pst[ps0 + e], n = pst[ps0 + e + 1] - x0;
            if (u < base + n) return c * kChunk + perm[x0 + u - base];
            base += n;
        }
        return 0;
    };
    Online st;
    st.init();
    // INT4: the group's mean rows (this lane's 8 elements) and the unit's code rows
    const int64_t qrow0 = ubase * kChunk;
    uint4 mk = make_uint4(0, 0, 0, 0), mv = mk;
    if constexpr (Q4) {
        const int64_t g = ubase * A.G + gid;
        mk = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(A.index + A.L.gk) + g * kD + 8 * l16);
        mv = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(A.index + A.L.gv) + g * kD + 8 * l16);
    }
    auto decode8 = [&](uint32_t code, float sc, const uint4& mean, float* f) {
        float mf[8];
        Elt<bf16_t>::unpack(mean, mf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int q = (int)((code >> (4 * e)) & 0xfu);
            f[e] = __builtin_fmaf(sc, (float)((q ^ 8) - 8), mf[e]);
        }
    };
    constexpr int RB = 12;  // rows in flight per batch (kept packed): most pairs need one batch
    for (int u0 = 0; u0 < nrow; u0 += RB) {
        const int pos = l16 < RB && u0 + l16 < nrow ? row_pos(u0 + l16) : 0;  // lane u: row u0 + u
        uint4 kp[RB], vp[RB];      // bf16 rows (packed)
        uint32_t kq[RB], vq[RB];   // INT4: codes of this lane's 8 elements
        float ks[RB], vs[RB];      // INT4: row scales
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            const int pu = __shfl(pos, seg0 + u, 64);
            if (u0 + u < nrow) {
                if constexpr (Q4) {
                    const int64_t row = qrow0 + pu;
                    kq[u] = *reinterpret_cast<const uint32_t*>(A.index + A.L.q4k + row * (kD / 2) + 4 * l16);
                    vq[u] = *reinterpret_cast<const uint32_t*>(A.index + A.L.q4v + row * (kD / 2) + 4 * l16);
                    ks[u] = reinterpret_cast<const float*>(A.index + A.L.q4ks)[row];
                    vs[u] = reinterpret_cast<const float*>(A.index + A.L.q4vs)[row];
                } else {
                    const int64_t ro = kv_pos<PAGED>(A, bs, pu);
                    kp[u] = *reinterpret_cast<const uint4*>(kc + ro + 8 * l16);
                    vp[u] = *reinterpret_cast<const uint4*>(vc + ro + 8 * l16);
                }
            }
        }
        // block update: dot products and their reductions side by side, one rescale
        float lam[RB];
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            float kf[8];
            if constexpr (Q4)
                decode8(kq[u], ks[u], mk, kf);
            else
                Elt<bf16_t>::unpack(kp[u], kf);
            float a = 0.0f;
#pragma unroll
            for (int z = 0; z < 8; ++z) a = __builtin_fmaf(q8[z], kf[z], a);
            lam[u] = a;
        }
#pragma unroll
        for (int u = 0; u < RB; ++u) lam[u] = row16_sum_f32(lam[u]);
        float mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            lam[u] = u0 + u < nrow ? A.scale * lam[u] : -INFINITY;
            mb = fmaxf(mb, lam[u]);
        }
        const float mn = fmaxf(st.m, mb);
        const float al = softmax_exp(st.m - mn);  // st.m = -inf -> 0
        st.l *= al;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.o[e] *= al;
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            if (lam[u] == -INFINITY) continue;  // no row: its registers were not loaded
            const float wgt = softmax_exp(lam[u] - mn);
            float vf[8];
            if constexpr (Q4)
                decode8(vq[u], vs[u], mv, vf);
            else
                Elt<bf16_t>::unpack(vp[u], vf);
            st.l += wgt;
#pragma unroll
            for (int e = 0; e < 8; ++e) st.o[e] = __builtin_fmaf(wgt, vf[e], st.o[e]);
        }
        st.m = mn;
    }
    // unopened pages: mean terms
    {
        uint32_t m = closed;
        for (; m; m &= m - 1) {
            const int e = __builtin_ctz(m);
            float vf[8];
            load8<bf16_t>(pv_u + ((int64_t)c * PS + ps0 + e) * kD, l16, vf);
            st.add(A.scale * __shfl(rl16, seg0 + e, 64) + __shfl(pln16, seg0 + e, 64), vf);
        }
    }
    float* dst = A.part_pg + (rh * A.TG + t) * kPartStride;
    *reinterpret_cast<float4*>(dst + 8 * l16) = make_float4(st.o[0], st.o[1], st.o[2], st.o[3]);
    *reinterpret_cast<float4*>(dst + 8 * l16 + 4) = make_float4(st.o[4], st.o[5], st.o[6], st.o[7]);
    if (l16 == 0) { dst[kD] = st.m; dst[kD + 1] = st.l; }
}

// ---------------------------------------------------------------------------- group pages (MFMA)

// The opened groups' pages on MFMA, group by group.  A workgroup takes kGroupPairs
// consecutive pairs of its unit's group-sorted list (one MFMA column each); the pairs
// form runs of equal group.  Up to kGroupRuns runs at a time share one key list: the
// members of each run's group in page order (K/V rows from the cache) and, when some pair
// leaves a page of the group unopened (more pages than top_pages, and a remainder), the
// group's page summaries (mean key and value, bias ln n).  A column sees a row of its own
// run: a member row when the row's page is opened for the pair, a summary row when it is
// not.  So each group's rows are read once per workgroup, not once per pair, and most
// workgroups need one key tile.  S^T = K Q^T and O^T = V^T P^T run as in the flash kernel
// (keys as MFMA rows, P from registers as bf16 hi + lo); each column's online softmax is
// written as the pair's partial state.  Four waves of one 16-column block each: 121
// registers, four waves per SIMD (two waves of two blocks each needed 222 registers and
// ran two per SIMD, 20% slower).
// Which runs share a workgroup depends on the order in which the bucket step filled the
// list, so a pair's result must not depend on its neighbours: a run's rows start at a
// 32-row boundary of a tile (the same positions of every 32-key MFMA sum wherever the run
// lands), a run never straddles tiles unless it has more than 64 rows (then it starts a
// tile of its own), and the rows of other runs enter only as exact zeros.
constexpr int kGroupThreads = 256;                  // four waves, one 16-column block each
constexpr int kGroupWaves = kGroupThreads / 64;
constexpr int kGroupPairs = 16 * kGroupWaves;       // pairs (MFMA columns) per workgroup
constexpr int kGroupRuns = 4;                       // runs sharing a key list (meta rows in LDS)
constexpr int kSumRow = 0x100;                      // flag of a summary row in GroupSmem::rpage

struct GroupSmem {
    alignas(16) bf16_t kt[kFlashKeys][kD];  // key tile
    alignas(16) bf16_t vt[kFlashKeys][kD];
    alignas(16) float bias[kFlashKeys];     // log2 units; -inf: no row
    alignas(16) int rpage[kFlashKeys];      // run << 16 | page of the row in its group (| kSumRow); -1: none
    int rsrc[kFlashKeys];                   // member: cache position; summary: unit page slot
    alignas(16) int16_t meta[kGroupRuns][kPagesMeta];  // meta rows of the batch's runs
    int2 ent[kGroupPairs];                  // (pair index, group) of the workgroup's pairs
    uint32_t open[kGroupPairs];             // opened-page mask of each pair
    int seg[kGroupPairs + 1];               // run starts (offsets into ent), then the end
    int runof[kGroupPairs];                 // run of each pair
    int rtile[kGroupRuns], roff[kGroupRuns], rn[kGroupRuns];  // placement of the batch's runs
    int ntile;                              // key tiles of the batch
    int firstrow, tilerows;                 // the tile's first row, 1 + its last row
    int nseg;
};

template <int HG, bool PAGED>
__global__ __launch_bounds__(kGroupThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void prefill_group_kernel(PagesArgs A) {
    __shared__ GroupSmem s;
    const int unit_local = blockIdx.y;
    const int qc = unit_local % A.units_per_seq_kv;
    const int kvh = (unit_local / A.units_per_seq_kv) % A.Hkv;
    const int b = unit_local / (A.units_per_seq_kv * A.Hkv);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
    const int64_t unit = unit_local;
    const int npairs = A.poff[unit * 2];
    const int x0 = blockIdx.x * kGroupPairs;
    if (x0 >= npairs) return;  // uniform in the workgroup
    const int np = min(kGroupPairs, npairs - x0);
    const int r0 = qc * kChunk;
    const int PS = A.L.page_slots;
    const int ms16 = A.L.meta_stride / 8;  // 16-byte pieces of a meta row
    const int2* list = A.plist + unit * (kChunk * HG * A.TG);
    const int bs = A.seq + b;
    const int64_t ubase = ((int64_t)bs * A.Hkv + kvh) * A.max_chunks;
    const int16_t* meta_u = reinterpret_cast<const int16_t*>(A.index + A.L.meta) + ubase * A.L.meta_stride;
    const bf16_t* pk_u = reinterpret_cast<const bf16_t*>(A.index + A.L.pk) + ubase * PS * kD;
    const bf16_t* pv_u = reinterpret_cast<const bf16_t*>(A.index + A.L.pv) + ubase * PS * kD;
    const float* pln_u = reinterpret_cast<const float*>(A.index + A.L.pln) + ubase * PS;
    const bf16_t* kc = A.k + kvh * A.sh + kv_seq<PAGED>(A, bs);
    const bf16_t* vc = A.v + kvh * A.sh + kv_seq<PAGED>(A, bs);
    const float sc2 = A.scale * kFlashLog2e;
    auto pair_rh = [&](int pi, int& t) {
        t = pi % A.TG;
        const int h = (pi / A.TG) % HG, rl = pi / (A.TG * HG);
        return ((int64_t)b * A.nq + r0 + rl) * A.Hq + kvh * HG + h;
    };
    auto load_metas = [&](int sb, int nrun) {  // meta rows of runs sb .. sb+nrun-1 -> slots 0..
        for (int x = tid; x < nrun * ms16; x += kGroupThreads) {
            const int k = x / ms16, e = x % ms16;
            const int c = s.ent[s.seg[sb + k]].y / A.G;
            *reinterpret_cast<uint4*>(&s.meta[k][8 * e]) =
                *reinterpret_cast<const uint4*>(meta_u + (int64_t)c * A.L.meta_stride + 8 * e);
        }
    };

    // the workgroup's pairs and the runs of equal group (wave 0: one pair per lane)
    if (w == 0) {
        const int2 e = l < np ? list[x0 + l] : make_int2(0, -1);
        s.ent[l] = e;
        const int prev = __shfl_up(e.y, 1, 64);
        const bool start = l < np && (l == 0 || e.y != prev);
        const uint64_t m = __ballot(start);
        const int below = __popcll(m & ((1ull << l) - 1ull));
        if (start) s.seg[below] = l;
        s.runof[l] = start ? below : below - 1;  // the run this pair belongs to
        if (l == 0) {
            s.nseg = __popcll(m);
            s.seg[__popcll(m)] = np;
        }
    }
    __syncthreads();
    const int nseg = s.nseg;
    // the pairs' opened-page masks and the first runs' meta rows, in one round trip; the
    // query operands of this lane's two columns are in flight meanwhile
    if (tid < kGroupPairs) {
        uint32_t op = 0;
        if (tid < np) {
            int t;
            const int64_t rh = pair_rh(s.ent[tid].x, t);
            op = A.rec[rh * A.TG + t].open;
        }
        s.open[tid] = op;
    }
    load_metas(0, min(nseg, kGroupRuns));
    // this lane's column: pair 16 w + li
    const int ncol = 16 * w + li;
    const bool cvalid = ncol < np;
    int ct;
    const int64_t crh = pair_rh(s.ent[cvalid ? ncol : 0].x, ct);
    bf16x8_t qb[4];
    {
        const bf16_t* qr = A.q + crh * kD;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qb[kk] = *reinterpret_cast<const bf16x8_t*>(qr + 32 * kk + 8 * g);
    }
    __syncthreads();
    const int crun = cvalid ? s.runof[ncol] : -1;
    const uint32_t copen = cvalid ? s.open[ncol] : 0u;

    for (int sb = 0; sb < nseg; sb += kGroupRuns) {  // batches of runs
        const int nrun = min(kGroupRuns, nseg - sb);
        if (sb > 0) {  // runs past the first batch (every use of the slots has ended)
            load_metas(sb, nrun);
            __syncthreads();
        }
        // rows of the batch's runs: members, then summaries if some pair of the run leaves
        // a page unopened (more pages than top_pages, and a remainder); placed in key tiles
        // at 32-row boundaries
        if (tid == 0) {
            int tile = 0, off = 0;
            for (int k = 0; k < nrun; ++k) {
                const int16_t* gpg = s.meta[k];
                const int16_t* pst = gpg + (A.G + 1);
                const int j = s.ent[s.seg[sb + k]].y % A.G;
                const int ps0 = gpg[j], npg = gpg[j + 1] - ps0;
                const bool sums = A.tp > 0 && npg > A.tp && !A.drop;
                const int n = pst[ps0 + npg] - pst[ps0] + (sums ? npg : 0);
                s.rn[k] = n;
                if (n > kFlashKeys) {  // its own tiles
                    if (off > 0) { ++tile; off = 0; }
                    s.rtile[k] = tile;
                    s.roff[k] = 0;
                    tile += (n + kFlashKeys - 1) / kFlashKeys;
                } else {
                    const int need = (n + 31) & ~31;
                    if (off + need > kFlashKeys) { ++tile; off = 0; }
                    s.rtile[k] = tile;
                    s.roff[k] = off;
                    off += need;
                    if (off == kFlashKeys) { ++tile; off = 0; }
                }
            }
            s.ntile = tile + (off > 0 ? 1 : 0);
        }
        __syncthreads();
        const int ntile = s.ntile;
        f32x4_t O[8];
        float m_run = -INFINITY, l_run = 0.0f;
#pragma unroll
        for (int db = 0; db < 8; ++db) O[db] = {0.0f, 0.0f, 0.0f, 0.0f};
        // the column's run in this batch (run sb + k is k here); a wave with none only
        // helps load
        const int cbat = (crun >= sb && crun < sb + nrun) ? crun - sb : -1;
        const bool active = __any(cbat >= 0);
        for (int kt = 0; kt < ntile; ++kt) {
            // the tile's rows: run k's members (cache position, page) then its summaries
            // (unit page slot, page | flag); -1: no row
            if (tid < kFlashKeys) {
                int k = -1, u = 0;
                for (int x = 0; x < nrun; ++x) {
                    const int o = (kt - s.rtile[x]) * kFlashKeys + tid - s.roff[x];
                    if (kt >= s.rtile[x] && o >= 0 && o < s.rn[x]) { k = x; u = o; }
                }
                int src = 0, pg = -1;
                float bias = -INFINITY;
                if (k >= 0) {
                    const int16_t* gpg = s.meta[k];
                    const int16_t* pst = gpg + (A.G + 1);
                    const int16_t* perm = pst + (PS + 1);
                    const int gid = s.ent[s.seg[sb + k]].y;
                    const int c = gid / A.G, j = gid % A.G;
                    const int ps0 = gpg[j], npg = gpg[j + 1] - ps0;
                    const int m0 = pst[ps0], nmem = pst[ps0 + npg] - m0;
                    if (u < nmem) {
                        const int x = m0 + u;
                        int e = 0;
                        while (e + 1 < npg && pst[ps0 + e + 1] <= x) ++e;
                        src = c * kChunk + perm[x];
                        pg = (k << 16) | e;
                        bias = 0.0f;
                    } else {
                        const int e = u - nmem;
                        src = c * PS + ps0 + e;
                        pg = (k << 16) | kSumRow | e;
                        bias = pln_u[src] * kFlashLog2e;
                    }
                }
                s.rsrc[tid] = src;
                s.rpage[tid] = pg;
                s.bias[tid] = bias;
                if (tid == 0) {  // the rows the tile spans
                    int first = kFlashKeys, last = 0;
                    for (int x = 0; x < nrun; ++x) {
                        const int o = (kt - s.rtile[x]) * kFlashKeys;  // rows of run x before this tile
                        if (kt < s.rtile[x] || o >= s.rn[x] + s.roff[x]) continue;
                        const int lo = kt == s.rtile[x] ? s.roff[x] : 0;
                        first = min(first, lo);
                        last = max(last, min(kFlashKeys, s.roff[x] + s.rn[x] - o));
                    }
                    s.firstrow = first;
                    s.tilerows = last;
                }
            }
            __syncthreads();
            const int nk = s.tilerows;
            // K and V rows straight into LDS (a wave's 64 lanes fill four rows per
            // instruction; a slot without a row loads the tile's first row, a valid
            // address, and is masked).  Every row's source is read from LDS before the
            // first load is issued: an LDS read after a load into LDS is made to wait for
            // it, which ran the four steps one after another.
            constexpr int kSteps = kFlashKeys / 4 / kGroupWaves;
            const bf16_t* ksrc[kSteps];
            const bf16_t* vsrc[kSteps];
            const int fr = s.firstrow;
#pragma unroll
            for (int ii = 0; ii < kSteps; ++ii) {
                const int row = 4 * (w + kGroupWaves * ii) + g;
                const int rr = s.rpage[row] >= 0 ? row : fr;
                const int src = s.rsrc[rr];
                const bool sum = (s.rpage[rr] & kSumRow) != 0;
                ksrc[ii] = sum ? pk_u + (int64_t)src * kD : kc + kv_pos<PAGED>(A, bs, src);
                vsrc[ii] = sum ? pv_u + (int64_t)src * kD : vc + kv_pos<PAGED>(A, bs, src);
            }
#pragma unroll
            for (int ii = 0; ii < kSteps; ++ii) {
                const int i = w + kGroupWaves * ii;
                const int row = 4 * i + g;
                __builtin_amdgcn_global_load_lds(ksrc[ii] + 8 * (li ^ fswz_k(row)), &s.kt[4 * i][0], 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vsrc[ii] + 8 * (li ^ fswz_v(row)), &s.vt[4 * i][0], 16, 0, 0);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (active) {
                const int nkb = (nk + 15) / 16;
                f32x4_t S[4];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    S[kb] = {0.0f, 0.0f, 0.0f, 0.0f};
                    if (kb < nkb) {
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) {
                            const int row = 16 * kb + li;
                            const int chunk = (4 * kk + g) ^ fswz_k(row);
                            const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&s.kt[row][8 * chunk]);
                            S[kb] = mfma16(av, qb[kk], S[kb]);
                        }
                    }
                }
                // logits (log2 units) of the column's own run under its page mask, online
                // softmax (a column's keys live in lanes l, l^16, l^32, l^48)
                float P[4][4];
                {
                    float mt = -INFINITY;
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        // a lane's four keys' tags and biases in one 16-byte read each (every
                        // slot written) and a branch-free mask
                        const int k4 = 16 * kb + 4 * g;
                        const int4 pg4 = *reinterpret_cast<const int4*>(&s.rpage[k4]);
                        float4 bi4 = *reinterpret_cast<const float4*>(&s.bias[k4]);
                        // through empty asm: otherwise the compiler splits the read and sinks
                        // each part into the mask's branch, where it is waited for alone
                        asm volatile("" : "+v"(bi4.x), "+v"(bi4.y), "+v"(bi4.z), "+v"(bi4.w));
                        const int pgr[4] = {pg4.x, pg4.y, pg4.z, pg4.w};
                        const float bir[4] = {bi4.x, bi4.y, bi4.z, bi4.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int pg = pgr[r];
                            const bool mine = (pg >= 0) & ((pg >> 16) == cbat);
                            const bool opened = ((copen >> (pg & 31)) & 1u) != 0;
                            const bool ok = mine & (((pg & kSumRow) != 0) != opened);
                            const float lam = ok ? __builtin_fmaf(sc2, S[kb][r], bir[r]) : -INFINITY;
                            P[kb][r] = lam;
                            mt = fmaxf(mt, lam);
                        }
                    }
                    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
                    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
                    const float mn = fmaxf(m_run, mt);
                    const float al = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mn);
                    const float ms = mn == -INFINITY ? 0.0f : mn;
                    float ls = 0.0f;
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float pw = __builtin_amdgcn_exp2f(P[kb][r] - ms);  // exp2(-inf) = 0
                            P[kb][r] = pw;
                            ls += pw;
                        }
                    l_run = __builtin_fmaf(l_run, al, ls);
                    m_run = mn;
                    if (__any(al != 1.0f)) {
#pragma unroll
                        for (int db = 0; db < 8; ++db) O[db] *= al;
                    }
                }
                // O^T += V^T P^T over the tile's 32-key steps (P as bf16 hi + lo)
#pragma unroll
                for (int sp = 0; sp < 2; ++sp) {
                    if (32 * sp >= nk) break;
                    bf16x8_t ph, pl;
#pragma unroll
                    for (int jj = 0; jj < 8; jj += 2) {
                        const ff32x2_t xv = {P[2 * sp + jj / 4][jj % 4], P[2 * sp + jj / 4][jj % 4 + 1]};
                        const fbf16x2_t h = __builtin_convertvector(xv, fbf16x2_t);
                        const ff32x2_t rv = xv - __builtin_convertvector(h, ff32x2_t);
                        const fbf16x2_t lo = __builtin_convertvector(rv, fbf16x2_t);
                        ph[jj] = h[0];
                        ph[jj + 1] = h[1];
                        pl[jj] = lo[0];
                        pl[jj + 1] = lo[1];
                    }
#pragma unroll
                    for (int db = 0; db < 8; ++db) {
                        const fs16x4_t v0 = flash_vt_read(s.vt, 32 * sp + 4 * g, 16 * db, li);
                        const fs16x4_t v1 = flash_vt_read(s.vt, 32 * sp + 16 + 4 * g, 16 * db, li);
                        const fs16x4_t both[2] = {v0, v1};
                        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, both);
                        O[db] = mfma16(av, ph, O[db]);
                        O[db] = mfma16(av, pl, O[db]);
                    }
                }
            }
            __syncthreads();  // the tile's rows are consumed before the next tile or batch
        }
        // the batch's columns: partial states (o, m in natural units, l)
        if (active) {
            float lt = l_run;
            lt += __shfl_xor(lt, 16, 64);
            lt += __shfl_xor(lt, 32, 64);
            if (cbat >= 0) {
                float* dst = A.part_pg + (crh * A.TG + ct) * kPartStride;
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    const f32x4_t o = O[db];
                    *reinterpret_cast<float4*>(dst + 16 * db + 4 * g) = make_float4(o[0], o[1], o[2], o[3]);
                }
                if (g == 0) {
                    dst[kD] = m_run == -INFINITY ? -INFINITY : m_run * kFlashLn2;
                    dst[kD + 1] = lt;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------- combine

// out = merge of the flash partial and the page partials of every opened slot.
// KM: the most states a call has (flash splits + page slots), so that the registers
// holding them in flight are no more than needed (with room for 24 states the kernel ran
// at two waves per SIMD).
template <int KM>
__global__ __launch_bounds__(kThreads) void prefill_combine_kernel(PagesArgs A, int64_t nrh) {
    // 32 threads per (row, head), 4 output elements each: 8 (row, head) per workgroup
    const int64_t rh = (int64_t)blockIdx.x * (kThreads / 32) + (threadIdx.x >> 5);
    const int d4 = 4 * (threadIdx.x & 31);
    if (rh >= nrh) return;
    // every state's (m, l, o[d4 .. d4+3]) loaded together: the flash splits, then the
    // page slots.  Slots past the last state load state 0 again and are dropped after the
    // loads (a load behind a branch would be waited for before the next one issues).
    constexpr int kMax = KM;
    const int nst = A.nsplit + A.TG;
    float mm[kMax], ll[kMax];
    float4 oo[kMax];
#pragma unroll
    for (int k = 0; k < kMax; ++k) {
        const float* pp = k < A.nsplit ? A.part_fl + k * A.split_stride + rh * kPartStride
                                       : A.part_pg + (rh * A.TG + (k - A.nsplit)) * kPartStride;  // empty slots hold m = -inf
        if (k >= nst) pp = A.part_fl + rh * kPartStride;
        const float2 ml = *reinterpret_cast<const float2*>(pp + kD);
        mm[k] = k < nst ? ml.x : -INFINITY;
        ll[k] = ml.y;
        oo[k] = *reinterpret_cast<const float4*>(pp + d4);
    }
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMax; ++k) M = fmaxf(M, mm[k]);
    float L = 0.0f, O0 = 0.0f, O1 = 0.0f, O2 = 0.0f, O3 = 0.0f;
#pragma unroll
    for (int k = 0; k < kMax; ++k) {
        if (mm[k] == -INFINITY) continue;
        const float e = softmax_exp(mm[k] - M);
        L = __builtin_fmaf(ll[k], e, L);
        O0 = __builtin_fmaf(oo[k].x, e, O0);
        O1 = __builtin_fmaf(oo[k].y, e, O1);
        O2 = __builtin_fmaf(oo[k].z, e, O2);
        O3 = __builtin_fmaf(oo[k].w, e, O3);
    }
    *reinterpret_cast<float4*>(A.out + rh * kD + d4) = make_float4(O0 / L, O1 / L, O2 / L, O3 / L);
}

}  // namespace lodi

// ---------------------------------------------------------------------------- host side

namespace lodi {

// Rows per prefill batch (a multiple of the chunk size): bounds the workspace.
constexpr int kPrefillBatchRows = 2048;

struct PrefillPlan {
    int rows;    // rows per batch (<= n_q, multiple of kChunk unless n_q is smaller)
    int nsplit;  // candidate sweeps and flash workgroups per (tile, KV head): enough
                 // workgroups for small batches
    size_t off_selg, off_rec, off_pfl, off_ppg, off_plist, off_poff, off_ltop, off_lcnt, off_lent, bytes;
};

// Workspace of one batch of rows of one sequence (sequences run one after another).
static PrefillPlan plan_prefill(const lod_params* p, int n_q) {
    PrefillPlan P{};
    P.rows = n_q < kPrefillBatchRows ? n_q : kPrefillBatchRows;
    const size_t rh = (size_t)P.rows * p->n_q_heads;
    const size_t TG = p->top_groups;
    const int HG = p->n_q_heads / p->n_kv_heads;
    const size_t units = (size_t)p->n_kv_heads * ((P.rows + kChunk - 1) / kChunk);
    const int64_t tiles = ((int64_t)P.rows * HG + kFlashRowHeads - 1) / kFlashRowHeads * p->n_kv_heads;
    int64_t ns = (512 + tiles - 1) / tiles;
    P.nsplit = (int)(ns < 1 ? 1 : (ns > 8 ? 8 : ns));
    size_t o = 0;
    P.off_selg = o; o = align256(o + rh * TG * 4);
    P.off_rec = o; o = align256(o + rh * TG * sizeof(PairRec));
    P.off_pfl = o; o = align256(o + (size_t)P.nsplit * rh * kPartStride * 4);
    P.off_ppg = o; o = align256(o + rh * TG * kPartStride * 4);
    P.off_plist = o; o = align256(o + units * kChunk * HG * TG * 8);
    P.off_poff = o; o = align256(o + units * 2 * 4);
    P.off_ltop = o; o = align256(o + (size_t)P.nsplit * rh * kMaxTG * 4);
    P.off_lcnt = o; o = align256(o + (size_t)P.nsplit * rh * 4);
    P.off_lent = o; o = align256(o + (size_t)P.nsplit * rh * kSplitCap * 8);
    P.bytes = o;
    return P;
}

template <int HG>
static int launch_prefill_batch(const SelArgs& S, const FlashArgs& F, const PagesArgs& P, int batch,
                                int nunits_q, hipStream_t st) {
    constexpr int QT = kFlashRowHeads / HG;
    const int ntiles = (S.nq + QT - 1) / QT;
    trace_point(0, st);
    // lane lists of 4 (8 for more than 8 opened groups): 16 (32) values per column;
    // launches of fewer than four workgroups per CU score whole tiles at a time
    const int64_t ncand = (int64_t)ntiles * S.nsplit * S.Hkv * batch;
    const dim3 gc(ntiles * S.nsplit * S.Hkv, 1, batch);
    if (ncand < 4 * kCUs) {
        if (S.TG <= 8) hipLaunchKernelGGL((prefill_cand_kernel<HG, 4, true>), gc, dim3(kThreads), 0, st, S);
        else hipLaunchKernelGGL((prefill_cand_kernel<HG, 8, true>), gc, dim3(kThreads), 0, st, S);
    } else {
        if (S.TG <= 8) hipLaunchKernelGGL((prefill_cand_kernel<HG, 4, false>), gc, dim3(kThreads), 0, st, S);
        else hipLaunchKernelGGL((prefill_cand_kernel<HG, 8, false>), gc, dim3(kThreads), 0, st, S);
    }
    trace_point(1, st);
    // half-size column groups where full ones would leave CUs with less than two
    // workgroups (the select steps are chains of dependent loads)
    // (sorting networks of 8 entries when at most 8 groups are opened)
    {
        const bool half = (int64_t)ntiles * (kFlashRowHeads / kSelCols) * S.Hkv * batch < 2 * kCUs;
        const dim3 gs(ntiles * (kFlashRowHeads / (half ? kSelCols / 2 : kSelCols)) * S.Hkv, 1, batch);
        if (half) {
            if (S.TG <= 8) hipLaunchKernelGGL((prefill_select_kernel<HG, kSelCols / 2, 8>), gs, dim3(kThreads), 0, st, S);
            else hipLaunchKernelGGL((prefill_select_kernel<HG, kSelCols / 2, kMaxTG>), gs, dim3(kThreads), 0, st, S);
        } else {
            if (S.TG <= 8) hipLaunchKernelGGL((prefill_select_kernel<HG, kSelCols, 8>), gs, dim3(kThreads), 0, st, S);
            else hipLaunchKernelGGL((prefill_select_kernel<HG, kSelCols, kMaxTG>), gs, dim3(kThreads), 0, st, S);
        }
    }
    trace_point(2, st);
    // flash and bucket in one launch when the bucket side's 512 threads hold a unit's pairs
    // in at most 32 slots each (HG * TG <= 64); else two launches
    const int per_fused = (kChunk * HG * S.TG + kFlashThreads - 1) / kFlashThreads;
    if (per_fused <= 32) {
        const int nflash = ntiles * F.nsplit * S.Hkv;
        const dim3 gf(nflash + nunits_q * S.Hkv, 1, batch);
        if (F.btab) {
            if (per_fused <= 16)
                hipLaunchKernelGGL((prefill_flash_bucket_kernel<HG, true, 16>), gf, dim3(kFlashThreads), 0, st, F, P, nflash,
                                   nunits_q);
            else
                hipLaunchKernelGGL((prefill_flash_bucket_kernel<HG, true, 32>), gf, dim3(kFlashThreads), 0, st, F, P, nflash,
                                   nunits_q);
        } else {
            if (per_fused <= 16)
                hipLaunchKernelGGL((prefill_flash_bucket_kernel<HG, false, 16>), gf, dim3(kFlashThreads), 0, st, F, P, nflash,
                                   nunits_q);
            else
                hipLaunchKernelGGL((prefill_flash_bucket_kernel<HG, false, 32>), gf, dim3(kFlashThreads), 0, st, F, P, nflash,
                                   nunits_q);
        }
        trace_point(3, st);
    } else {
        if (F.btab)
            hipLaunchKernelGGL((prefill_flash_kernel<HG, true>), dim3(ntiles * F.nsplit, S.Hkv, batch), dim3(kFlashThreads),
                               0, st, F);
        else
            hipLaunchKernelGGL((prefill_flash_kernel<HG, false>), dim3(ntiles * F.nsplit, S.Hkv, batch), dim3(kFlashThreads),
                               0, st, F);
        trace_point(3, st);
        const dim3 gb(nunits_q, S.Hkv, batch);
        const int per = (kChunk * HG * S.TG + kBucketThreads - 1) / kBucketThreads;
        if (per <= 4) hipLaunchKernelGGL((prefill_bucket_kernel<HG, 4>), gb, dim3(kBucketThreads), 0, st, P);
        else if (per <= 8) hipLaunchKernelGGL((prefill_bucket_kernel<HG, 8>), gb, dim3(kBucketThreads), 0, st, P);
        else if (per <= 16) hipLaunchKernelGGL((prefill_bucket_kernel<HG, 16>), gb, dim3(kBucketThreads), 0, st, P);
        else hipLaunchKernelGGL((prefill_bucket_kernel<HG, 32>), gb, dim3(kBucketThreads), 0, st, P);
    }
    trace_point(4, st);
    const int maxpairs = kChunk * HG * S.TG;
    const dim3 pgrid((maxpairs + kPairsPerWG - 1) / kPairsPerWG, nunits_q * S.Hkv * batch);
    const dim3 ggrid((maxpairs + kGroupPairs - 1) / kGroupPairs, nunits_q * S.Hkv * batch);
    if (P.q4)  // decoded from the index (not bf16 rows): the VALU kernel; the view does not matter
        hipLaunchKernelGGL((prefill_pages_kernel<HG, false, true>), pgrid, dim3(kThreads), 0, st, P);
    else if (P.btab)
        hipLaunchKernelGGL((prefill_group_kernel<HG, true>), ggrid, dim3(kGroupThreads), 0, st, P);
    else
        hipLaunchKernelGGL((prefill_group_kernel<HG, false>), ggrid, dim3(kGroupThreads), 0, st, P);
    trace_point(5, st);
    const int64_t nrh = (int64_t)batch * S.nq * S.Hq;
    const dim3 cgrid((unsigned)((nrh + kThreads / 32 - 1) / (kThreads / 32)));
    const int nstates = P.nsplit + P.TG;
    if (nstates <= 9)
        hipLaunchKernelGGL((prefill_combine_kernel<9>), cgrid, dim3(kThreads), 0, st, P, nrh);
    else if (nstates <= 12)
        hipLaunchKernelGGL((prefill_combine_kernel<12>), cgrid, dim3(kThreads), 0, st, P, nrh);
    else if (nstates <= 16)
        hipLaunchKernelGGL((prefill_combine_kernel<16>), cgrid, dim3(kThreads), 0, st, P, nrh);
    else
        hipLaunchKernelGGL((prefill_combine_kernel<8 + kMaxTG>), cgrid, dim3(kThreads), 0, st, P, nrh);
    trace_point(6, st);
    return LOD_OK;
}

}  // namespace lodi

namespace lodi {

template <int HG>
static void launch_flash(const FlashArgs& A, int batch, hipStream_t st) {
    constexpr int QT = kFlashRowHeads / HG;
    if (A.btab)
        hipLaunchKernelGGL((prefill_flash_kernel<HG, true>), dim3((A.nq + QT - 1) / QT, A.Hkv, batch), dim3(kFlashThreads),
                           0, st, A);
    else
        hipLaunchKernelGGL((prefill_flash_kernel<HG, false>), dim3((A.nq + QT - 1) / QT, A.Hkv, batch), dim3(kFlashThreads),
                           0, st, A);
}

static int dispatch_flash(const FlashArgs& A, int batch, hipStream_t st) {
    switch (A.Hq / A.Hkv) {
        case 1: launch_flash<1>(A, batch, st); break;
        case 2: launch_flash<2>(A, batch, st); break;
        case 4: launch_flash<4>(A, batch, st); break;
        default: launch_flash<8>(A, batch, st); break;
    }
    return hipGetLastError() == hipSuccess ? LOD_OK : LOD_ERR_HIP;
}

}  // namespace lodi

using namespace lodi;

extern "C" int lod_dense_prefill(const lod_params* params, lod_kv kv, const void* q, int32_t q_start,
                                 int32_t n_q, int32_t batch, float* out, void* stream) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!q || !out || batch <= 0 || n_q <= 0 || q_start < 0) return LOD_ERR_ARG;
    if (!aligned16(q) || !aligned16(out)) return LOD_ERR_ARG;
    if ((rc = check_kv_view(params, kv, (int64_t)q_start + n_q)) != LOD_OK) return rc;
    if ((int64_t)q_start + n_q > INT32_MAX) return LOD_ERR_ARG;
    if (params->kv_dtype != LOD_BF16)
        return dense_prefill_valu(params, kv, q, q_start, n_q, batch, out, stream);
    FlashArgs A{};
    A.k = reinterpret_cast<const bf16_t*>(kv.k);
    A.v = reinterpret_cast<const bf16_t*>(kv.v);
    set_kv_map(A, kv);
    A.q = reinterpret_cast<const bf16_t*>(q);
    A.nq = n_q; A.pos0 = q_start;
    A.Hq = params->n_q_heads; A.Hkv = params->n_kv_heads; A.scale = params->scale;
    A.index = nullptr;
    A.out = out;
    return dispatch_flash(A, batch, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int lod_prefill_ws_bytes(const lod_params* params, int32_t batch, int32_t n_q,
                                    int32_t max_tokens, size_t* bytes) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!bytes || batch <= 0 || n_q <= 0 || max_tokens <= 0) return LOD_ERR_ARG;
    if (params->kv_dtype != LOD_BF16) return prefill_rows_ws_bytes(params, n_q, max_tokens, bytes);
    *bytes = plan_prefill(params, n_q).bytes;
    return LOD_OK;
}

extern "C" int lod_attend_prefill(const lod_params* params, const lod_index* index, lod_kv kv,
                                  const void* q, int32_t q_start, int32_t n_q, int32_t batch,
                                  float* out, int32_t* sel_groups, int32_t* sel_pages, void* ws,
                                  size_t ws_bytes, void* stream) {
    int rc = check_params(params);
    if (rc != LOD_OK) return rc;
    if (!index || !index->mem || !q || !out || batch <= 0 || n_q <= 0 || q_start < 0) return LOD_ERR_ARG;
    if (!aligned16(q) || !aligned16(out)) return LOD_ERR_ARG;
    if (q_start % params->chunk_size != 0) return LOD_ERR_ARG;
    if ((rc = check_kv_view(params, kv, (int64_t)q_start + n_q)) != LOD_OK) return rc;
    if (batch != index->batch) return LOD_ERR_ARG;
    const int64_t end = (int64_t)q_start + n_q;
    if (end > INT32_MAX || built_chunks(params, end - 1) > index->max_chunks) return LOD_ERR_ARG;
    const lod_index_layout_t L = make_layout(params, index->batch, index->max_chunks);
    if (index->bytes < L.total) return LOD_ERR_WORKSPACE;
    if (params->kv_dtype != LOD_BF16)
        return prefill_rows(params, index, kv, q, q_start, n_q, batch, out, sel_groups, sel_pages, ws,
                            ws_bytes, stream);
    if ((int64_t)built_chunks(params, end - 1) * params->groups_per_chunk > kMaxBucketGroups)
        return LOD_ERR_UNSUPPORTED;
    const PrefillPlan P = plan_prefill(params, n_q);
    if (!ws || ws_bytes < P.bytes) return LOD_ERR_WORKSPACE;
    char* w = reinterpret_cast<char*>(ws);
    const int Hq = params->n_q_heads, Hkv = params->n_kv_heads, HG = Hq / Hkv, TG = params->top_groups;
    const int TPW = params->top_pages > 0 ? params->top_pages : 1;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    for (int r0 = 0; r0 < n_q; r0 += P.rows) {
        const int rows = (n_q - r0) < P.rows ? (n_q - r0) : P.rows;
        const int nunits_q = (rows + kChunk - 1) / kChunk;
        // batch rows are taken from every sequence: q rows [r0, r0+rows) of each b
        for (int b = 0; b < batch; ++b) {
            const int64_t row0 = (int64_t)b * n_q + r0;
            SelArgs S{};
            S.q = reinterpret_cast<const bf16_t*>(q) + row0 * Hq * kD;
            S.nq = rows; S.pos0 = q_start + r0; S.Hq = Hq; S.Hkv = Hkv;
            S.index = reinterpret_cast<const char*>(index->mem);
            S.L = L; S.max_chunks = index->max_chunks; S.G = params->groups_per_chunk;
            S.W = params->window; S.TG = TG; S.TP = params->top_pages;
            S.sel_groups = sel_groups ? sel_groups + row0 * Hq * TG : nullptr;
            S.sel_pages = sel_pages ? sel_pages + row0 * Hq * TG * TPW : nullptr;
            S.selg = reinterpret_cast<int32_t*>(w + P.off_selg);
            S.rec = reinterpret_cast<PairRec*>(w + P.off_rec);
            S.part_pg = reinterpret_cast<float*>(w + P.off_ppg);
            S.nsplit = P.nsplit;
            S.ltop = reinterpret_cast<float*>(w + P.off_ltop);
            S.lcnt = reinterpret_cast<int32_t*>(w + P.off_lcnt);
            S.lent = reinterpret_cast<uint2*>(w + P.off_lent);
            S.seq = b;
            FlashArgs F{};
            F.k = reinterpret_cast<const bf16_t*>(kv.k);
            F.v = reinterpret_cast<const bf16_t*>(kv.v);
            F.seq = b;
            set_kv_map(F, kv);
            F.q = S.q; F.nq = rows; F.pos0 = S.pos0; F.Hq = Hq; F.Hkv = Hkv; F.scale = params->scale;
            F.index = S.index; F.L = L; F.max_chunks = S.max_chunks; F.G = S.G; F.W = S.W;
            F.n_sink = params->n_sink; F.TG = TG; F.selg = S.selg; F.drop = params->drop_remainder;
            F.part = reinterpret_cast<float*>(w + P.off_pfl);
            F.nsplit = P.nsplit;
            F.split_stride = (int64_t)P.rows * Hq * kPartStride;
            PagesArgs G{};
            G.k = F.k; G.v = F.v; G.seq = b;
            set_kv_map(G, kv);
            G.q = S.q; G.nq = rows; G.pos0 = S.pos0; G.Hq = Hq; G.Hkv = Hkv; G.scale = params->scale;
            G.index = S.index; G.L = L; G.max_chunks = S.max_chunks; G.G = S.G; G.W = S.W; G.TG = TG;
            G.drop = params->drop_remainder;
            G.q4 = params->int4_pages;
            G.tp = params->top_pages;
            G.rec = S.rec;
            G.selg = S.selg;
            G.plist = reinterpret_cast<int2*>(w + P.off_plist);
            G.poff = reinterpret_cast<int32_t*>(w + P.off_poff);
            G.part_fl = F.part;
            G.nsplit = F.nsplit;
            G.split_stride = F.split_stride;
            G.part_pg = reinterpret_cast<float*>(w + P.off_ppg);
            G.out = out + row0 * Hq * kD;
            G.units_per_seq_kv = nunits_q;
            switch (HG) {
                case 1: rc = launch_prefill_batch<1>(S, F, G, 1, nunits_q, st); break;
                case 2: rc = launch_prefill_batch<2>(S, F, G, 1, nunits_q, st); break;
                case 4: rc = launch_prefill_batch<4>(S, F, G, 1, nunits_q, st); break;
                default: rc = launch_prefill_batch<8>(S, F, G, 1, nunits_q, st); break;
            }
            if (rc != LOD_OK) return rc;
        }
        if (hipGetLastError() != hipSuccess) return LOD_ERR_HIP;
    }
    return LOD_OK;
}
