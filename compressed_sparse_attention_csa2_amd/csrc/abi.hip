// C ABI of the CSA2 layer: argument validation, workspace layout and kernel
// launches on the caller's stream.  Declarations and the contract of every
// entry point are in include/csa2.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "csa2.h"
#include "csa2_device.h"

namespace csa2 {
__global__ void k_compress(int, int, const int32_t*, const uint16_t*, const uint16_t*,
                           const float*, const uint16_t*, const float*, const uint16_t*,
                           const float*, const float*, int64_t, uint8_t*, uint8_t*, uint8_t*,
                           uint8_t*, int64_t, int, int);
__global__ void k_window_encode(int, int, const int32_t*, const uint16_t*, const float*,
                                const float*, int64_t, uint8_t*, float*, int);
__global__ void k_append(int, const int32_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                         uint16_t*, uint16_t*, const float*, const uint16_t*, const float*,
                         const uint16_t*, const float*, const float*, int64_t, uint8_t*, uint8_t*,
                         uint8_t*, uint8_t*, int64_t, uint8_t*, float*, int, int, int);
__global__ void k_encode_fp4_rows(const uint16_t*, int64_t, int, uint8_t*, uint8_t*);
__global__ void k_encode_fp8_rows(const uint16_t*, int64_t, int, uint8_t*, float*);
__global__ void k_encode_fp4e4_rows(const uint16_t*, int64_t, int, uint8_t*, uint8_t*);
__global__ void k_decode_fp4e4_rows(const uint8_t*, const uint8_t*, int64_t, int, uint16_t*);
__global__ void k_attn_dq(int, int, int, const int32_t*, const uint16_t*, const uint8_t*,
                          const float*, int, const uint8_t*, const uint8_t*, int64_t,
                          const int32_t*, const int32_t*, const float*, const float*,
                          const float*, int64_t, uint16_t*, float*, const int32_t*, int, float*,
                          float*);
__global__ void k_decode_fp4_rows(const uint8_t*, const uint8_t*, int64_t, int, uint16_t*);
__global__ void k_decode_fp8_rows(const uint8_t*, int64_t, int, uint16_t*);
__global__ void k_prefill_entries(int, int, const int32_t*, int64_t, int32_t*, int);
__global__ void k_quant_index_query(const uint16_t*, const float*, int64_t, uint8_t*, float*);
template <int TOK>
__global__ void k_index_scores(int, int, const int32_t*, const int32_t*, const uint8_t*,
                               const float*, const uint8_t*, const uint8_t*, int64_t, float*,
                               int64_t, int, int, int);
__global__ void k_topk(int, int, const int32_t*, const int32_t*, const float*, int64_t, int64_t,
                       int, int, int32_t*, int32_t*, uint32_t*, int32_t*, int32_t*, uint32_t*,
                       const int32_t*, int);
__global__ void k_block_keys(int, int, const int32_t*, const int32_t*, int64_t, const float*,
                             int64_t, uint32_t*, int64_t, int);
__global__ void k_pool_select(int, int, const int32_t*, const int32_t*, int64_t, const uint32_t*,
                              int64_t, int32_t*, int32_t*, int);
__global__ void k_pool_scores(int, int, const int32_t*, const int32_t*, const uint8_t*,
                              const float*, const uint8_t*, const uint8_t*, int64_t,
                              const int32_t*, const int32_t*, float*, int64_t, int32_t*, int);
__global__ void k_pool_map(int64_t, const int32_t*, int32_t*);
__global__ void k_topk_merge(int, int, const uint32_t*, const int32_t*, const int32_t*,
                             const uint32_t*, int32_t*, int32_t*);
__global__ void k_topk_row(int, int, const int32_t*, const int32_t*, const float*, int64_t,
                           int64_t, int32_t*, int32_t*, int, const int32_t*);
template <int TOK>
__global__ void k_index_select(int, int, const int32_t*, const int32_t*, const uint8_t*,
                               const float*, const uint8_t*, const uint8_t*, int64_t, int, int,
                               int, int, int32_t*, int32_t*, uint32_t*, int32_t*, int32_t*,
                               uint32_t*, uint32_t*);
__global__ void k_zero_u32(uint32_t*, int64_t);
__global__ void k_fs_threshold(int, int, const int32_t*, const int32_t*, const uint16_t*,
                               const float*, uint8_t*, float*, const uint8_t*, const uint8_t*,
                               int64_t, int, uint32_t*);
__global__ void k_fs_scan(int, const int32_t*, const int32_t*, const uint8_t*, const float*,
                          const uint8_t*, const uint8_t*, int64_t, int, int, int, const uint32_t*,
                          uint32_t*, int32_t*, int32_t*);
template <int NT>
__global__ void k_fs_scan_nt(int, int, const int32_t*, const int32_t*, const uint8_t*,
                             const float*, const uint8_t*, const uint8_t*, int64_t, int, int, int,
                             const uint32_t*, uint32_t*, int32_t*, int32_t*);
__global__ void k_fs_select(int, int, const int32_t*, const int32_t*, const uint8_t*, const float*,
                            const uint8_t*, const uint8_t*, int64_t, int, int, int,
                            const uint32_t*, const uint32_t*, const int32_t*, const int32_t*,
                            int32_t*, int32_t*);
__global__ void k_z_fp8_rows(int64_t, const uint8_t*, const uint8_t*, uint8_t*, float*);
template <int HG, bool ZF8>
__global__ void k_attn(int, int, int, const int32_t*, const uint16_t*, const uint8_t*,
                       const float*, int, const uint8_t*, const uint8_t*, int64_t, const int32_t*,
                       const int32_t*, const float*, const float*, const float*, int64_t,
                       uint16_t*, float*, int, float*, float*, const int32_t*, int);
__global__ void k_attn_combine(int, int, int, const int32_t*, const float*, const float*,
                               const float*, int64_t, int, const float*, const float*, uint16_t*,
                               float*);
}  // namespace csa2

using namespace csa2;

// Scratch of csa2_index_topk_noalloc: one array per GPU, part of the library's
// code object.  In host code `scratch` only names the symbol; its device address
// comes from hipGetSymbolAddress (scratch_ptr below).
static __device__ __align__(256) uint8_t scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

csa2_status fail(csa2_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

csa2_status ok() {
    g_err[0] = 0;
    return CSA2_OK;
}

csa2_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CSA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return CSA2_OK;
}

inline hipStream_t S(void* s) { return (hipStream_t)s; }

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int MAX_ROWS = WINDOW + TOPK;

int index_tok(int Tq) { return Tq == 1 ? 1 : (Tq <= 8 ? 8 : 4); }

// Compute units of the current device, queried once per device.  The cache is
// atomic: concurrent first calls may both query, and both store the same value.
int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cus[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
            v = 256;
        cus[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Device address of the current device's scratch array, looked up on the first
// call per device (with that device current) and kept; concurrent first calls
// store the same address.  NULL (and an error message) if the lookup fails.
void* scratch_ptr() {
    static std::atomic<void*> ptrs[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        fail(CSA2_ERR_HIP, "scratch: no current device (%s)", hipGetErrorString(e));
        return nullptr;
    }
    void* p = ptrs[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            fail(CSA2_ERR_HIP, "scratch: hipGetSymbolAddress failed (%s)", hipGetErrorString(e));
            return nullptr;
        }
        ptrs[dev].store(p, std::memory_order_release);
    }
    return p;
}

// split of a token's attention rows (20 chunks of 32 at full size) across
// blocks when there are too few tokens to fill the chip.  The persistent
// kernel (k_attn) takes one block per token from 128 tokens on (B=128 decode:
// 33 us, against 28 us + a 9 us merge of the partials with two splits); the
// dequantising kernel (k_attn_dq, one block of four waves per unit) from 256.
int attn_split(int64_t tokens, bool dq = false) {
    if (tokens >= (dq ? 256 : 128)) return 1;
    // k_attn is persistent (one block per compute unit): no more units than
    // blocks, so that no block takes two (96 verify rows: 2 splits, not 3)
    const int64_t t1 = tokens > 0 ? tokens : 1;
    const int ns = (int)(dq ? cdiv(256, t1) : 256 / t1);
    return ns > 8 ? 8 : ns;
}

// Segments per query row for the selection: enough lists (one wave each) to
// fill the chip when rows are few, at most 32 segments of at least 8192 entries
// (96 rows over 524,288 entries: 32 segments 455 us, 16 559 us, 48 or 64
// 480-488 us; B=128 decode over 65,536 entries: 8 segments beat 16 and 4).
int topk_segments(int64_t rows, int64_t stride) {
    int64_t ns = cdiv(8192, rows > 0 ? rows : 1);
    if (ns > 32) ns = 32;
    const int64_t by_len = stride / 8192;
    if (ns > by_len) ns = by_len;
    return ns < 1 ? 1 : (int)ns;
}
int topk_seg_len(int64_t stride, int nseg) { return (int)(cdiv(cdiv(stride, nseg), 256) * 256); }
int64_t score_pitch(int64_t stride) { return cdiv(stride, 64) * 64; }   // floats between score rows

struct IndexWs {
    size_t q8, wq, S, seg_key, seg_j, seg_n, seg_kth, total;
};
IndexWs index_ws(int B, int Tq, int64_t stride) {
    IndexWs w;
    const size_t rows = (size_t)B * Tq;
    const int nseg = topk_segments((int64_t)rows, stride);
    w.q8 = 0;
    w.wq = align256(rows * HI * DI);
    w.S = w.wq + align256(rows * HI * sizeof(float));
    w.seg_key = w.S + align256(rows * (size_t)score_pitch(stride) * sizeof(float));
    const size_t segc = nseg > 1 ? rows * nseg * TOPK : 0;
    w.seg_j = w.seg_key + align256(segc * sizeof(uint32_t));
    w.seg_n = w.seg_j + align256(segc * sizeof(int32_t));
    w.seg_kth = w.seg_n + align256((nseg > 1 ? rows * nseg : 0) * sizeof(int32_t));
    w.total = w.seg_kth + align256((nseg > 1 ? rows * nseg * 2 : 0) * sizeof(uint32_t));
    return w;
}

// Full-layer selection with the hierarchical pool: the index workspace, then
// the block keys [rows][ceil(stride / 8)].
struct PoolWs {
    IndexWs ix;
    size_t keys, total;
    int64_t kpad;
};
PoolWs pool_ws(int B, int Tq, int64_t stride) {
    PoolWs w;
    w.ix = index_ws(B, Tq, stride);
    w.kpad = cdiv(cdiv(stride, 8), 4) * 4;   // rows of keys 16-byte aligned
    w.keys = w.ix.total;
    w.total = w.keys + align256((size_t)B * Tq * (size_t)w.kpad * sizeof(uint32_t));
    return w;
}
// Reindex: an index workspace for lists of the pool's 16,384 candidates, then
// the lists' lengths [rows].
constexpr int64_t POOL_CAND = (int64_t)POOL_BLOCKS * 8;
struct ReindexWs {
    IndexWs ix;
    size_t len, total;
};
ReindexWs reindex_ws(int B, int Tq) {
    ReindexWs w;
    w.ix = index_ws(B, Tq, POOL_CAND);
    w.len = w.ix.total;
    w.total = w.len + align256((size_t)B * Tq * sizeof(int32_t));
    return w;
}

// Fused scores + selection: the quantised queries, and when rows are cut into
// segments, the segments' winners and one arrival counter per row.  Rows are
// cut so that about 2,048 waves scan (segments of at least 4,096 entries, at
// most 64 per row) and no segment exceeds 65,536 entries.
struct SelWs {
    int tok, n_tg, nseg, seg_len;
    size_t q8, wq, seg_key, seg_j, seg_n, seg_kth, done, total;
};
SelWs select_ws(int B, int Tq, int64_t stride) {
    SelWs w;
    const size_t rows = (size_t)B * Tq;
    w.tok = index_tok(Tq);
    w.n_tg = (int)cdiv(Tq, w.tok);
    const int64_t groups = (int64_t)B * w.n_tg;
    int64_t ns = groups < 2048 ? cdiv(2048, groups) : 1;
    if (ns > 64) ns = 64;
    if (ns > stride / 4096) ns = stride / 4096;
    if (ns < cdiv(stride, 65536)) ns = cdiv(stride, 65536);   // entry offsets are 16-bit
    if (ns < 1) ns = 1;
    w.seg_len = (int)(cdiv(cdiv(stride, ns), 64) * 64);
    w.nseg = (int)cdiv(stride, w.seg_len);
    w.q8 = 0;
    w.wq = align256(rows * HI * DI);
    w.seg_key = w.wq + align256(rows * HI * sizeof(float));
    const size_t segc = w.nseg > 1 ? rows * w.nseg * TOPK : 0;
    w.seg_j = w.seg_key + align256(segc * sizeof(uint32_t));
    w.seg_n = w.seg_j + align256(segc * sizeof(int32_t));
    w.seg_kth = w.seg_n + align256((w.nseg > 1 ? rows * w.nseg : 0) * sizeof(int32_t));
    w.done = w.seg_kth + align256((w.nseg > 1 ? rows * w.nseg * 2 : 0) * sizeof(uint32_t));
    w.total = w.done + align256((w.nseg > 1 ? rows : 0) * sizeof(uint32_t));
    return w;
}

bool two_pass_rows(int B, int Tq, int64_t stride);

// Decode rows (one to eight tokens a request) over long caches: a sampled
// threshold, a scan that keeps only the keys at or above it (wcap slots per
// chunk of IDX_CHUNK entries, in entry order) and a cut of those; no score row.
// The threshold aims at about 2,048 candidates a row, about 2^22 / stride a
// chunk: wcap = 2^26 / stride (16 times that) between 64 and 512 slots.
bool fs_rows(int B, int Tq, int64_t stride) { return Tq <= 8 && two_pass_rows(B, Tq, stride); }
struct FsWs {
    int n_ch, wcap;
    size_t q8, wq, th, ccnt, ck, cj, total;
};
FsWs fs_ws(int B, int Tq, int64_t stride) {
    FsWs w;
    const size_t rows = (size_t)B * Tq;
    w.n_ch = (int)cdiv(stride, IDX_CHUNK);
    const int64_t wc = ((int64_t)1 << 26) / stride;
    w.wcap = (int)(wc < 64 ? 64 : (wc > 512 ? 512 : wc));
    const size_t slots = rows * (size_t)w.n_ch * w.wcap;
    w.q8 = 0;
    w.wq = align256(rows * HI * DI);
    w.th = w.wq + align256(rows * HI * sizeof(float));
    w.ccnt = w.th + align256(rows * sizeof(uint32_t));
    w.ck = w.ccnt + align256(rows * (size_t)w.n_ch * sizeof(int32_t));
    w.cj = w.ck + align256(slots * sizeof(uint32_t));
    w.total = w.cj + align256(slots * sizeof(int32_t));
    return w;
}

size_t index_topk_ws(int B, int Tq, int64_t stride) {
    if (fs_rows(B, Tq, stride)) return fs_ws(B, Tq, stride).total;
    return two_pass_rows(B, Tq, stride) ? index_ws(B, Tq, stride).total
                                        : select_ws(B, Tq, stride).total;
}

// Attention reads the compressed rows re-encoded as E4M3 rows with an fp32 row
// scale (k_z_fp8_rows, once per call) when the call gathers each entry of the
// caches at least four times on average (Tq * 512 >= 4 * entry_stride: a
// prefill), and the re-encoded rows stay within the kernel's 32-bit offsets.
bool attn_zf8(int B, int Tq, int64_t stride) {
    return (int64_t)Tq * TOPK >= 4 * stride && stride * 512 <= (int64_t)0xFFFFFFFF &&
           (int64_t)B * stride <= ((int64_t)1 << 26);
}

struct AttnWs {
    int nsplit, nsplit_dq, hsplit;
    bool zf8;
    size_t pO, pml, zq, zs, total;
};
// (the partials are sized for the larger split count of the two kernels)
AttnWs attn_ws(int B, int Tq, int H, int64_t stride) {
    AttnWs w;
    // k_attn: 65 to 128 query rows fill the GPU with two head groups a row (no
    // merge: heads are independent) in place of row splits and their merge
    const int64_t rows = (int64_t)B * Tq;
    w.hsplit = (H % 32 == 0 && rows > 64 && rows <= 128) ? 2 : 1;
    w.nsplit = w.hsplit > 1 ? 1 : attn_split(rows);
    w.nsplit_dq = attn_split(rows, true);
    w.zf8 = attn_zf8(B, Tq, stride);
    w.pO = 0;
    w.pml = 0;
    w.total = 0;
    const int ns = w.nsplit > w.nsplit_dq ? w.nsplit : w.nsplit_dq;
    if (ns > 1) {
        const size_t n = (size_t)B * Tq * ns * H;
        w.pml = align256(n * D * sizeof(float));
        w.total = w.pml + align256(n * 2 * sizeof(float));
    }
    w.zq = w.total;
    w.zs = w.zq;
    if (w.zf8) {
        const size_t ne = (size_t)B * (size_t)stride;
        w.zs = w.zq + align256(ne * D);
        w.total = w.zs + align256(ne * sizeof(float));
    }
    return w;
}

// positions per compressed entry: 2 (pooled pairs) or 1 (one entry per
// position); the kernels take its log2
bool bad_ratio(int ratio) { return ratio != 1 && ratio != 2; }

// compressed-row storage: 0 = one E8M0 scale per 32 channels (16 scale bytes per
// entry), 1 = the pages' one E4M3 scale per 16 channels (32 scale bytes)
bool bad_zfmt(int z_format) { return z_format != 0 && z_format != 1; }

bool bad_sizes(int B, int Tq, int64_t stride) {
    return B < 1 || Tq < 0 || stride < 1 || (int64_t)B * Tq > (int64_t)0x7FFFFFFF;
}

void launch_scores(int B, int Tq, const int32_t* q_pos0, const int32_t* n_entries,
                   const uint16_t* qI, const float* wI, const uint8_t* ki_codes,
                   const uint8_t* ki_scales, int64_t stride, float* Sc, int64_t s_stride, int rsh,
                   void* ws, hipStream_t st) {
    const IndexWs L = index_ws(B, Tq, stride);
    uint8_t* base = (uint8_t*)ws;
    uint8_t* q8 = base + L.q8;
    float* wq = (float*)(base + L.wq);
    const int64_t qrows = (int64_t)B * Tq * HI;
    hipLaunchKernelGGL(k_quant_index_query, dim3((unsigned)cdiv(qrows, 16)), dim3(256), 0, st, qI,
                       wI, qrows, q8, wq);
    const int tok = index_tok(Tq);
    const int n_tg = (int)cdiv(Tq, tok);
    const int n_ch = (int)cdiv(stride, IDX_CHUNK);
    const int64_t items = (int64_t)B * n_tg * n_ch;
    // four items per block; with four tokens per wave a block holds four token
    // groups of one chunk, so the groups are padded to a multiple of four
    const dim3 grid((unsigned)(tok == 4 ? (int64_t)B * cdiv(n_tg, 4) * n_ch : cdiv(items, 4)));
    if (tok == 1)
        hipLaunchKernelGGL(k_index_scores<1>, grid, dim3(256), 0, st, B, Tq, q_pos0, n_entries, q8,
                           wq, ki_codes, ki_scales, stride, Sc, s_stride, n_tg, n_ch, rsh);
    else if (tok == 8)
        hipLaunchKernelGGL(k_index_scores<8>, grid, dim3(256), 0, st, B, Tq, q_pos0, n_entries, q8,
                           wq, ki_codes, ki_scales, stride, Sc, s_stride, n_tg, n_ch, rsh);
    else
        hipLaunchKernelGGL(k_index_scores<4>, grid, dim3(256), 0, st, B, Tq, q_pos0, n_entries, q8,
                           wq, ki_codes, ki_scales, stride, Sc, s_stride, n_tg, n_ch, rsh);
}

// Few long rows (the decode and verify shapes): scores to the workspace and a
// selection pass win there.  Measured at 128 single-token rows of 65,536
// entries: 161 us for the two passes against 210 us fused (16 segments a row,
// each from a sampled threshold, then a merge); the fused scan alone, without
// the merge, took 190 us -- two waves a SIMD streaming the keys with the
// admission work of every tile keep it below the score pass's bandwidth.
bool two_pass_rows(int B, int Tq, int64_t stride) {
    return (int64_t)B * Tq <= 1024 && stride >= 16384;
}

csa2_status launch_index_2pass(int B, int Tq, const int32_t* q_pos0, const int32_t* n_entries,
                               const uint16_t* qI, const float* wI, const uint8_t* ki_codes,
                               const uint8_t* ki_scales, int64_t stride, int rsh, int32_t* idx,
                               int32_t* cnt, void* ws, hipStream_t st);

// Scores and selection in one kernel: no score row is written (csa2_index_topk,
// csa2_forward), except for few long rows (two_pass_rows).
csa2_status launch_index(int B, int Tq, const int32_t* q_pos0, const int32_t* n_entries,
                         const uint16_t* qI, const float* wI, const uint8_t* ki_codes,
                         const uint8_t* ki_scales, int64_t stride, int rsh, int32_t* idx,
                         int32_t* cnt, void* ws, hipStream_t st) {
    if (Tq == 0) return CSA2_OK;
    if (fs_rows(B, Tq, stride)) {
        const FsWs L = fs_ws(B, Tq, stride);
        uint8_t* base = (uint8_t*)ws;
        uint8_t* q8 = base + L.q8;
        float* wq = (float*)(base + L.wq);
        uint32_t* th = (uint32_t*)(base + L.th);
        int32_t* ccnt = (int32_t*)(base + L.ccnt);
        uint32_t* ck = (uint32_t*)(base + L.ck);
        int32_t* cj = (int32_t*)(base + L.cj);
        const int rows = B * Tq;
        hipLaunchKernelGGL(k_fs_threshold, dim3((unsigned)rows), dim3(512), 0, st, B, Tq, q_pos0,
                           n_entries, qI, wI, q8, wq, ki_codes, ki_scales, stride, rsh, th);
        const dim3 sgrid((unsigned)cdiv((int64_t)B * L.n_ch, 4));
        if (Tq == 1)
            hipLaunchKernelGGL(k_fs_scan, sgrid, dim3(256), 0, st, B, q_pos0, n_entries, q8, wq,
                               ki_codes, ki_scales, stride, L.n_ch, rsh, L.wcap,
                               (const uint32_t*)th, ck, cj, ccnt);
        else {
#define CSA2_FSN(NT)                                                                           \
    hipLaunchKernelGGL((k_fs_scan_nt<NT>), sgrid, dim3(256), 0, st, B, Tq, q_pos0, n_entries, q8, \
                       wq, ki_codes, ki_scales, stride, L.n_ch, rsh, L.wcap, (const uint32_t*)th, \
                       ck, cj, ccnt)
            switch (Tq) {
                case 2: CSA2_FSN(2); break;
                case 3: CSA2_FSN(3); break;
                case 4: CSA2_FSN(4); break;
                case 5: CSA2_FSN(5); break;
                case 6: CSA2_FSN(6); break;
                case 7: CSA2_FSN(7); break;
                default: CSA2_FSN(8); break;
            }
#undef CSA2_FSN
        }
        hipLaunchKernelGGL(k_fs_select, dim3((unsigned)rows), dim3(512), 0, st, B, Tq, q_pos0,
                           n_entries, q8, wq, ki_codes, ki_scales, stride, L.n_ch, rsh, L.wcap,
                           (const uint32_t*)th, (const uint32_t*)ck, (const int32_t*)cj,
                           (const int32_t*)ccnt, idx, cnt);
        return check_launch("csa2_index_topk");
    }
    if (two_pass_rows(B, Tq, stride))
        return launch_index_2pass(B, Tq, q_pos0, n_entries, qI, wI, ki_codes, ki_scales, stride,
                                  rsh, idx, cnt, ws, st);
    const SelWs L = select_ws(B, Tq, stride);
    uint8_t* base = (uint8_t*)ws;
    uint8_t* q8 = base + L.q8;
    float* wq = (float*)(base + L.wq);
    uint32_t* seg_key = (uint32_t*)(base + L.seg_key);
    int32_t* seg_j = (int32_t*)(base + L.seg_j);
    int32_t* seg_n = (int32_t*)(base + L.seg_n);
    uint32_t* seg_kth = (uint32_t*)(base + L.seg_kth);
    uint32_t* done = (uint32_t*)(base + L.done);
    const int64_t rows = (int64_t)B * Tq;
    const int64_t qrows = rows * HI;
    hipLaunchKernelGGL(k_quant_index_query, dim3((unsigned)cdiv(qrows, 16)), dim3(256), 0, st, qI,
                       wI, qrows, q8, wq);
    if (L.nseg > 1)
        hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)cdiv(rows, 256)), dim3(256), 0, st, done, rows);
    const int64_t items = (int64_t)B * L.n_tg * L.nseg;
    if (items > (int64_t)0x7FFFFFFF) return fail(CSA2_ERR_SHAPE, "index_topk: too many rows");
#define CSA2_SEL(T)                                                                            \
    hipLaunchKernelGGL(k_index_select<T>, dim3((unsigned)items), dim3(64), 0, st, B, Tq, q_pos0, \
                       n_entries, q8, wq, ki_codes, ki_scales, stride, L.n_tg, L.nseg,          \
                       L.seg_len, rsh, idx, cnt, seg_key, seg_j, seg_n, seg_kth, done)
    if (L.tok == 1) CSA2_SEL(1);
    else if (L.tok == 8) CSA2_SEL(8);
    else CSA2_SEL(4);
#undef CSA2_SEL
    return check_launch("csa2_index_topk");
}

// Scores written to the workspace, then a selection pass over them (the pool
// needs every score for its block keys).
csa2_status launch_index_2pass(int B, int Tq, const int32_t* q_pos0, const int32_t* n_entries,
                               const uint16_t* qI, const float* wI, const uint8_t* ki_codes,
                               const uint8_t* ki_scales, int64_t stride, int rsh, int32_t* idx,
                               int32_t* cnt, void* ws, hipStream_t st) {
    if (Tq == 0) return CSA2_OK;
    const IndexWs L = index_ws(B, Tq, stride);
    float* Sc = (float*)((uint8_t*)ws + L.S);
    const int64_t pitch = score_pitch(stride);
    launch_scores(B, Tq, q_pos0, n_entries, qI, wI, ki_codes, ki_scales, stride, Sc, pitch, rsh, ws,
                  st);
    const int64_t rows = (int64_t)B * Tq;
    if (rows <= 1024 && stride >= 16384 && stride <= 131072) {
        // few rows of moderate length: one block per row, no segments to merge
        hipLaunchKernelGGL(k_topk_row, dim3((unsigned)rows), dim3(512), 0, st, B, Tq, q_pos0,
                           n_entries, Sc, pitch, stride, idx, cnt, rsh, (const int32_t*)nullptr);
        return check_launch("csa2_index_topk");
    }
    const int nseg = topk_segments(rows, stride);
    const int seg_len = topk_seg_len(stride, nseg);
    uint32_t* seg_key = (uint32_t*)((uint8_t*)ws + L.seg_key);
    int32_t* seg_j = (int32_t*)((uint8_t*)ws + L.seg_j);
    int32_t* seg_n = (int32_t*)((uint8_t*)ws + L.seg_n);
    uint32_t* seg_kth = (uint32_t*)((uint8_t*)ws + L.seg_kth);
    hipLaunchKernelGGL(k_topk, dim3((unsigned)cdiv(rows * nseg, 4)), dim3(256), 0, st, B, Tq,
                       q_pos0, n_entries, Sc, pitch, stride, nseg, seg_len, idx, cnt, seg_key,
                       seg_j, seg_n, seg_kth, (const int32_t*)nullptr, rsh);
    if (nseg > 1)
        hipLaunchKernelGGL(k_topk_merge, dim3((unsigned)cdiv(rows, 4)), dim3(256), 0, st,
                           (int)rows, nseg, seg_key, seg_j, seg_n, seg_kth, idx, cnt);
    return check_launch("csa2_index_topk");
}

csa2_status launch_attn(int B, int Tq, int H, const int32_t* q_pos0, const uint16_t* Q,
                        const uint8_t* w_codes, const float* w_scale, int cap,
                        const uint8_t* z_codes, const uint8_t* z_scales, int64_t stride,
                        int z_format, const int32_t* idx, const int32_t* cnt, const float* sink,
                        const float* rc, const float* rs, int64_t rope_rows, uint16_t* O,
                        float* lse, const int32_t* win_floor, void* ws, hipStream_t st) {
    if (Tq == 0) return CSA2_OK;
    if (z_format == 1) {
        // rows in the pages' format: the dequantising kernel, one block per (query,
        // split); the splits' partials are merged as on the per-32 path
        const AttnWs L = attn_ws(B, Tq, H, stride);
        float* pO = (float*)((uint8_t*)ws + L.pO);
        float* pml = (float*)((uint8_t*)ws + L.pml);
        const int64_t units = (int64_t)B * Tq * L.nsplit_dq;
        if (units > (int64_t)0x7FFFFFFF) return fail(CSA2_ERR_SHAPE, "sparse_attn: too many rows");
        hipLaunchKernelGGL(k_attn_dq, dim3((unsigned)units), dim3(256), 0, st, B, Tq, H, q_pos0,
                           Q, w_codes, w_scale, cap, z_codes, z_scales, stride, idx, cnt, sink,
                           rc, rs, rope_rows, O, lse, win_floor, L.nsplit_dq, pO, pml);
        if (L.nsplit_dq > 1) {
            const int64_t items = (int64_t)B * Tq * H;
            hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)cdiv(items, 4)), dim3(256), 0, st,
                               B, Tq, H, q_pos0, sink, rc, rs, rope_rows, L.nsplit_dq, pO, pml, O,
                               lse);
        }
        return check_launch("csa2_sparse_attn");
    }
    // the kernel addresses one request's caches with 32-bit byte offsets
    if ((int64_t)cap * D > (int64_t)0xFFFFFFFF || stride * 256 > (int64_t)0xFFFFFFFF)
        return fail(CSA2_ERR_RANGE, "sparse_attn: cap=%d (at most 8388607) or entry stride=%lld "
                    "(at most 16777215) too large", cap, (long long)stride);
    const AttnWs L = attn_ws(B, Tq, H, stride);
    float* pO = (float*)((uint8_t*)ws + L.pO);
    float* pml = (float*)((uint8_t*)ws + L.pml);
    if (L.zf8) {
        // the compressed rows in the window's format (E4M3 + fp32 row scale)
        uint8_t* zq = (uint8_t*)ws + L.zq;
        float* zsf = (float*)((uint8_t*)ws + L.zs);
        const int64_t ne = (int64_t)B * stride;
        hipLaunchKernelGGL(k_z_fp8_rows, dim3((unsigned)cdiv(ne, 8)), dim3(256), 0, st, ne,
                           z_codes, z_scales, zq, zsf);
        z_codes = zq;
        z_scales = (const uint8_t*)zsf;
    }
    // persistent blocks (one per compute unit) walk the (row, split, head group) units
    const int64_t units = (int64_t)B * Tq * L.nsplit * L.hsplit;
    if (units > (int64_t)0x7FFFFFFF) return fail(CSA2_ERR_SHAPE, "sparse_attn: too many rows");
    const int64_t nblk = units < device_cus() ? units : device_cus();
    const dim3 grid((unsigned)nblk);
    const int ht = H / 16 / L.hsplit;   // head tiles of 16 a unit
#define CSA2_ATTN(HTV, ZF)                                                                     \
    hipLaunchKernelGGL((k_attn<HTV, ZF>), grid, dim3(ATT_THREADS), 0, st, B, Tq, H, q_pos0, Q,     \
                       w_codes, w_scale, cap, z_codes, z_scales, stride, idx, cnt, sink, rc, rs,   \
                       rope_rows, O, lse, L.nsplit, pO, pml, win_floor, L.hsplit)
    if (L.zf8) {
        switch (ht) {
            case 1: CSA2_ATTN(1, true); break;
            case 2: CSA2_ATTN(2, true); break;
            case 3: CSA2_ATTN(3, true); break;
            default: CSA2_ATTN(4, true); break;
        }
    } else {
        switch (ht) {
            case 1: CSA2_ATTN(1, false); break;
            case 2: CSA2_ATTN(2, false); break;
            case 3: CSA2_ATTN(3, false); break;
            default: CSA2_ATTN(4, false); break;
        }
    }
#undef CSA2_ATTN
    if (L.nsplit > 1) {
        const int64_t items = (int64_t)B * Tq * H;
        hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)cdiv(items, 4)), dim3(256), 0, st, B,
                           Tq, H, q_pos0, sink, rc, rs, rope_rows, L.nsplit, pO, pml, O, lse);
    }
    return check_launch("csa2_sparse_attn");
}

}  // namespace

extern "C" {

int csa2_abi_version(void) { return CSA2_ABI_VERSION; }

const char* csa2_last_error(void) { return g_err; }

const char* csa2_status_string(csa2_status s) {
    switch (s) {
        case CSA2_OK: return "ok";
        case CSA2_ERR_NULL: return "null pointer";
        case CSA2_ERR_SHAPE: return "bad shape";
        case CSA2_ERR_UNSUPPORTED: return "unsupported size";
        case CSA2_ERR_RANGE: return "buffer too small";
        case CSA2_ERR_WORKSPACE: return "workspace too small";
        case CSA2_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t csa2_workspace_size(int op, int B, int Tq, int H, int64_t entry_stride) {
    if (bad_sizes(B, Tq, entry_stride)) return 0;
    if (op == CSA2_OP_INDEX_TOPK) return index_topk_ws(B, Tq, entry_stride);
    if (op == CSA2_OP_INDEX_SCORES) return index_ws(B, Tq, entry_stride).S;
    if (op == CSA2_OP_INDEX_POOL) return pool_ws(B, Tq, entry_stride).total;
    if (op == CSA2_OP_REINDEX) return reindex_ws(B, Tq).total;
    if (H < 16 || H > 64 || H % 16) return 0;
    if (op == CSA2_OP_SPARSE_ATTN) return attn_ws(B, Tq, H, entry_stride).total;
    if (op == CSA2_OP_FORWARD) {
        size_t a = index_topk_ws(B, Tq, entry_stride), c = attn_ws(B, Tq, H, entry_stride).total;
        return (a > c ? a : c) + align256((size_t)B * sizeof(int32_t));
    }
    return 0;
}

csa2_status csa2_compress(int B, int T, const int32_t* pos0, const uint16_t* kc,
                          const uint16_t* gc, const float* gamma_c, const uint16_t* w_ik,
                          const float* gamma_ik, const uint16_t* ki_given, const float* rope_cos,
                          const float* rope_sin, int64_t rope_rows, uint8_t* z_codes,
                          uint8_t* z_scales, uint8_t* ki_codes, uint8_t* ki_scales,
                          int64_t entry_stride, int ratio, int z_format, void* stream) {
    if (bad_sizes(B, T, entry_stride)) return fail(CSA2_ERR_SHAPE, "compress: B=%d T=%d stride=%lld", B, T, (long long)entry_stride);
    if (bad_ratio(ratio)) return fail(CSA2_ERR_UNSUPPORTED, "compress: ratio=%d (need 1 or 2)", ratio);
    if (bad_zfmt(z_format)) return fail(CSA2_ERR_UNSUPPORTED, "compress: z_format=%d (need 0 or 1)", z_format);
    if (T == 0) return ok();     // no work: no pointer is read
    if (!pos0 || !kc || (ratio == 2 && !gc) || !gamma_c || !rope_cos || !rope_sin || !z_codes ||
        !z_scales || !ki_codes || !ki_scales)
        return fail(CSA2_ERR_NULL, "compress: a required pointer is NULL");
    if (w_ik ? !gamma_ik : !ki_given)
        return fail(CSA2_ERR_NULL, "compress: need w_ik+gamma_ik (derive) or ki_given (given)");
    if (rope_rows < 1) return fail(CSA2_ERR_RANGE, "compress: empty rotary table");
    const int rsh = ratio == 2 ? 1 : 0;
    const int64_t items = (int64_t)B * (T >> rsh);
    if (items == 0) return ok();
    hipLaunchKernelGGL(k_compress, dim3((unsigned)cdiv(items, 4)), dim3(256), 0, S(stream), B, T,
                       pos0, kc, gc, gamma_c, w_ik, gamma_ik, ki_given, rope_cos, rope_sin,
                       rope_rows, z_codes, z_scales, ki_codes, ki_scales, entry_stride, rsh,
                       z_format);
    csa2_status s = check_launch("csa2_compress");
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_encode_window(int B, int T, const int32_t* pos0, const uint16_t* wn,
                               const float* rope_cos, const float* rope_sin, int64_t rope_rows,
                               uint8_t* w_codes, float* w_scale, int cap, void* stream) {
    if (bad_sizes(B, T, 1) || cap < 1) return fail(CSA2_ERR_SHAPE, "encode_window: B=%d T=%d cap=%d", B, T, cap);
    if (T == 0) return ok();     // no work: no pointer is read
    if (!pos0 || !wn || !rope_cos || !rope_sin || !w_codes || !w_scale)
        return fail(CSA2_ERR_NULL, "encode_window: a required pointer is NULL");
    if (rope_rows < 1) return fail(CSA2_ERR_RANGE, "encode_window: empty rotary table");
    const int64_t items = (int64_t)B * T;
    if (items == 0) return ok();
    hipLaunchKernelGGL(k_window_encode, dim3((unsigned)cdiv(items, 4)), dim3(256), 0, S(stream),
                       B, T, pos0, wn, rope_cos, rope_sin, rope_rows, w_codes, w_scale, cap);
    csa2_status s = check_launch("csa2_encode_window");
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_append(int B, const int32_t* pos, const uint16_t* kc, const uint16_t* gc,
                        const uint16_t* wn, uint16_t* pair_kc, uint16_t* pair_gc,
                        const float* gamma_c, const uint16_t* w_ik, const float* gamma_ik,
                        const uint16_t* ki_given, const float* rope_cos, const float* rope_sin,
                        int64_t rope_rows, uint8_t* z_codes, uint8_t* z_scales,
                        uint8_t* ki_codes, uint8_t* ki_scales, int64_t entry_stride, int ratio,
                        int z_format, uint8_t* w_codes, float* w_scale, int cap, void* stream) {
    if (B < 0 || entry_stride < 1 || cap < 1)
        return fail(CSA2_ERR_SHAPE, "append: B=%d stride=%lld cap=%d", B, (long long)entry_stride, cap);
    if (bad_ratio(ratio)) return fail(CSA2_ERR_UNSUPPORTED, "append: ratio=%d (need 1 or 2)", ratio);
    if (bad_zfmt(z_format)) return fail(CSA2_ERR_UNSUPPORTED, "append: z_format=%d (need 0 or 1)", z_format);
    if (B == 0) return ok();     // no work: no pointer is read
    if (!pos || !kc || !wn || (ratio == 2 && (!gc || !pair_kc || !pair_gc)) || !gamma_c ||
        !rope_cos || !rope_sin || !z_codes || !z_scales || !ki_codes || !ki_scales || !w_codes ||
        !w_scale)
        return fail(CSA2_ERR_NULL, "append: a required pointer is NULL");
    if (w_ik ? !gamma_ik : !ki_given)
        return fail(CSA2_ERR_NULL, "append: need w_ik+gamma_ik (derive) or ki_given (given)");
    if (rope_rows < 1) return fail(CSA2_ERR_RANGE, "append: empty rotary table");
    if (B == 0) return ok();
    hipLaunchKernelGGL(k_append, dim3((unsigned)B), dim3(128), 0, S(stream), B, pos, kc, gc, wn,
                       pair_kc, pair_gc, gamma_c, w_ik, gamma_ik, ki_given, rope_cos, rope_sin,
                       rope_rows, z_codes, z_scales, ki_codes, ki_scales, entry_stride, w_codes,
                       w_scale, cap, ratio == 2 ? 1 : 0, z_format);
    csa2_status s = check_launch("csa2_append");
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_index_topk(int B, int Tq, const int32_t* q_pos0, const int32_t* n_entries,
                            const uint16_t* qI, const float* wI, const uint8_t* ki_codes,
                            const uint8_t* ki_scales, int64_t entry_stride, int ratio,
                            int32_t* idx, int32_t* cnt, void* ws, size_t ws_bytes,
                            void* stream) {
    if (bad_sizes(B, Tq, entry_stride)) return fail(CSA2_ERR_SHAPE, "index_topk: B=%d Tq=%d stride=%lld", B, Tq, (long long)entry_stride);
    if (bad_ratio(ratio)) return fail(CSA2_ERR_UNSUPPORTED, "index_topk: ratio=%d (need 1 or 2)", ratio);
    if (Tq == 0) return ok();     // no work: no pointer is read
    if (!q_pos0 || !n_entries || !qI || !wI || !ki_codes || !ki_scales || !idx || !cnt)
        return fail(CSA2_ERR_NULL, "index_topk: a required pointer is NULL");
    const size_t need = index_topk_ws(B, Tq, entry_stride);
    if (Tq > 0 && (!ws || ws_bytes < need))
        return fail(CSA2_ERR_WORKSPACE, "index_topk: workspace %zu < %zu bytes", ws_bytes, need);
    csa2_status s = launch_index(B, Tq, q_pos0, n_entries, qI, wI, ki_codes, ki_scales,
                                 entry_stride, ratio == 2 ? 1 : 0, idx, cnt, ws, S(stream));
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_index_topk_noalloc(int B, int Tq, const int32_t* q_pos0,
                                    const int32_t* n_entries, const uint16_t* qI,
                                    const float* wI, const uint8_t* ki_codes,
                                    const uint8_t* ki_scales, int64_t entry_stride, int ratio,
                                    int32_t* idx, int32_t* cnt, void* stream) {
    if (bad_sizes(B, Tq, entry_stride)) return fail(CSA2_ERR_SHAPE, "index_topk_noalloc: B=%d Tq=%d stride=%lld", B, Tq, (long long)entry_stride);
    if (bad_ratio(ratio)) return fail(CSA2_ERR_UNSUPPORTED, "index_topk_noalloc: ratio=%d (need 1 or 2)", ratio);
    if (Tq == 0) return ok();     // no work: no pointer is read
    if (!q_pos0 || !n_entries || !qI || !wI || !ki_codes || !ki_scales || !idx || !cnt)
        return fail(CSA2_ERR_NULL, "index_topk_noalloc: a required pointer is NULL");
    const size_t need = index_topk_ws(B, Tq, entry_stride);
    if (need > CSA2_NOALLOC_SCRATCH_BYTES)
        return fail(CSA2_ERR_WORKSPACE, "index_topk_noalloc: these sizes need %zu bytes of scratch, "
                    "more than the library's %zu", need, (size_t)CSA2_NOALLOC_SCRATCH_BYTES);
    void* ws = scratch_ptr();
    if (ws == nullptr) return CSA2_ERR_HIP;
    csa2_status s = launch_index(B, Tq, q_pos0, n_entries, qI, wI, ki_codes, ki_scales,
                                 entry_stride, ratio == 2 ? 1 : 0, idx, cnt, ws, S(stream));
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_index_pool(int B, int Tq, const int32_t* q_pos0, const int32_t* n_entries,
                            const uint16_t* qI, const float* wI, const uint8_t* ki_codes,
                            const uint8_t* ki_scales, int64_t entry_stride, int ratio,
                            int32_t* idx, int32_t* cnt, int32_t* pool, int32_t* pool_cnt,
                            void* ws, size_t ws_bytes, void* stream) {
    if (bad_sizes(B, Tq, entry_stride)) return fail(CSA2_ERR_SHAPE, "index_pool: B=%d Tq=%d stride=%lld", B, Tq, (long long)entry_stride);
    if (bad_ratio(ratio)) return fail(CSA2_ERR_UNSUPPORTED, "index_pool: ratio=%d (need 1 or 2)", ratio);
    const int rsh = ratio == 2 ? 1 : 0;
    if (Tq == 0) return ok();     // no work: no pointer is read
    if (!q_pos0 || !n_entries || !qI || !wI || !ki_codes || !ki_scales || !idx || !cnt || !pool ||
        !pool_cnt)
        return fail(CSA2_ERR_NULL, "index_pool: a required pointer is NULL");
    const PoolWs L = pool_ws(B, Tq, entry_stride);
    if (Tq > 0 && (!ws || ws_bytes < L.total))
        return fail(CSA2_ERR_WORKSPACE, "index_pool: workspace %zu < %zu bytes", ws_bytes, L.total);
    if (Tq == 0) return ok();
    hipStream_t st = S(stream);
    csa2_status s = launch_index_2pass(B, Tq, q_pos0, n_entries, qI, wI, ki_codes, ki_scales,
                                       entry_stride, rsh, idx, cnt, ws, st);
    if (s != CSA2_OK) return s;
    const float* Sc = (const float*)((uint8_t*)ws + L.ix.S);
    uint32_t* keys = (uint32_t*)((uint8_t*)ws + L.keys);
    const int64_t rows = (int64_t)B * Tq;
    hipLaunchKernelGGL(k_block_keys, dim3((unsigned)cdiv(rows * L.kpad, 256)), dim3(256), 0, st, B,
                       Tq, q_pos0, n_entries, entry_stride, Sc, score_pitch(entry_stride), keys,
                       L.kpad, rsh);
    hipLaunchKernelGGL(k_pool_select, dim3((unsigned)rows), dim3(256), 0, st, B, Tq, q_pos0,
                       n_entries, entry_stride, keys, L.kpad, pool, pool_cnt, rsh);
    s = check_launch("csa2_index_pool");
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_reindex_topk(int B, int Tq, const int32_t* q_pos0, const int32_t* n_entries,
                              const uint16_t* qI, const float* wI, const uint8_t* ki_codes,
                              const uint8_t* ki_scales, int64_t entry_stride, int ratio,
                              const int32_t* pool, const int32_t* pool_cnt, int32_t* idx,
                              int32_t* cnt, void* ws, size_t ws_bytes, void* stream) {
    if (bad_sizes(B, Tq, entry_stride)) return fail(CSA2_ERR_SHAPE, "reindex_topk: B=%d Tq=%d stride=%lld", B, Tq, (long long)entry_stride);
    if (bad_ratio(ratio)) return fail(CSA2_ERR_UNSUPPORTED, "reindex_topk: ratio=%d (need 1 or 2)", ratio);
    const int rsh = ratio == 2 ? 1 : 0;
    if (Tq == 0) return ok();     // no work: no pointer is read
    if (!q_pos0 || !n_entries || !qI || !wI || !ki_codes || !ki_scales || !pool || !pool_cnt ||
        !idx || !cnt)
        return fail(CSA2_ERR_NULL, "reindex_topk: a required pointer is NULL");
    const ReindexWs L = reindex_ws(B, Tq);
    if (Tq > 0 && (!ws || ws_bytes < L.total))
        return fail(CSA2_ERR_WORKSPACE, "reindex_topk: workspace %zu < %zu bytes", ws_bytes, L.total);
    if (Tq == 0) return ok();
    hipStream_t st = S(stream);
    uint8_t* base = (uint8_t*)ws;
    uint8_t* q8 = base + L.ix.q8;
    float* wq = (float*)(base + L.ix.wq);
    float* Sc = (float*)(base + L.ix.S);
    int32_t* len = (int32_t*)(base + L.len);
    const int64_t rows = (int64_t)B * Tq;
    const int64_t qrows = rows * HI;
    hipLaunchKernelGGL(k_quant_index_query, dim3((unsigned)cdiv(qrows, 16)), dim3(256), 0, st, qI,
                       wI, qrows, q8, wq);
    const int64_t pitch = score_pitch(POOL_CAND);
    hipLaunchKernelGGL(k_pool_scores, dim3((unsigned)cdiv(rows * (POOL_BLOCKS / 128), 4)),
                       dim3(256), 0, st, B, Tq, q_pos0, n_entries, q8, wq, ki_codes, ki_scales,
                       entry_stride, pool, pool_cnt, Sc, pitch, len, rsh);
    if (rows <= 1024) {
        // the pool lists (at most 16,384 scores each): one block per row
        hipLaunchKernelGGL(k_topk_row, dim3((unsigned)rows), dim3(512), 0, st, B, Tq, q_pos0,
                           n_entries, Sc, pitch, (int64_t)POOL_CAND, idx, cnt, rsh,
                           (const int32_t*)len);
        hipLaunchKernelGGL(k_pool_map, dim3((unsigned)cdiv(rows * TOPK, 256)), dim3(256), 0, st,
                           rows, pool, idx);
        csa2_status s = check_launch("csa2_reindex_topk");
        return s == CSA2_OK ? ok() : s;
    }
    const int nseg = topk_segments(rows, POOL_CAND);
    const int seg_len = topk_seg_len(POOL_CAND, nseg);
    uint32_t* seg_key = (uint32_t*)(base + L.ix.seg_key);
    int32_t* seg_j = (int32_t*)(base + L.ix.seg_j);
    int32_t* seg_n = (int32_t*)(base + L.ix.seg_n);
    uint32_t* seg_kth = (uint32_t*)(base + L.ix.seg_kth);
    hipLaunchKernelGGL(k_topk, dim3((unsigned)cdiv(rows * nseg, 4)), dim3(256), 0, st, B, Tq,
                       q_pos0, n_entries, Sc, pitch, POOL_CAND, nseg, seg_len, idx, cnt, seg_key,
                       seg_j, seg_n, seg_kth, (const int32_t*)len, rsh);
    if (nseg > 1)
        hipLaunchKernelGGL(k_topk_merge, dim3((unsigned)cdiv(rows, 4)), dim3(256), 0, st,
                           (int)rows, nseg, seg_key, seg_j, seg_n, seg_kth, idx, cnt);
    hipLaunchKernelGGL(k_pool_map, dim3((unsigned)cdiv(rows * TOPK, 256)), dim3(256), 0, st, rows,
                       pool, idx);
    csa2_status s = check_launch("csa2_reindex_topk");
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_index_scores(int B, int Tq, const int32_t* q_pos0, const int32_t* n_entries,
                              const uint16_t* qI, const float* wI, const uint8_t* ki_codes,
                              const uint8_t* ki_scales, int64_t entry_stride, int ratio,
                              float* scores, void* ws, size_t ws_bytes, void* stream) {
    if (bad_sizes(B, Tq, entry_stride)) return fail(CSA2_ERR_SHAPE, "index_scores: B=%d Tq=%d stride=%lld", B, Tq, (long long)entry_stride);
    if (bad_ratio(ratio)) return fail(CSA2_ERR_UNSUPPORTED, "index_scores: ratio=%d (need 1 or 2)", ratio);
    if (Tq == 0) return ok();     // no work: no pointer is read
    if (!q_pos0 || !n_entries || !qI || !wI || !ki_codes || !ki_scales || !scores)
        return fail(CSA2_ERR_NULL, "index_scores: a required pointer is NULL");
    const size_t need = index_ws(B, Tq, entry_stride).S;
    if (Tq > 0 && (!ws || ws_bytes < need))
        return fail(CSA2_ERR_WORKSPACE, "index_scores: workspace %zu < %zu bytes", ws_bytes, need);
    if (Tq == 0) return ok();
    launch_scores(B, Tq, q_pos0, n_entries, qI, wI, ki_codes, ki_scales, entry_stride, scores,
                  entry_stride, ratio == 2 ? 1 : 0, ws, S(stream));
    csa2_status s = check_launch("csa2_index_scores");
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_sparse_attn(int B, int Tq, int H, const int32_t* q_pos0, const uint16_t* Q,
                             const uint8_t* w_codes, const float* w_scale, int cap,
                             const uint8_t* z_codes, const uint8_t* z_scales, int64_t entry_stride,
                             int z_format, const int32_t* idx, const int32_t* cnt,
                             const float* sink, const float* rope_cos, const float* rope_sin,
                             int64_t rope_rows, uint16_t* O, float* lse, const int32_t* win_floor,
                             void* ws, size_t ws_bytes, void* stream) {
    if (bad_zfmt(z_format)) return fail(CSA2_ERR_UNSUPPORTED, "sparse_attn: z_format=%d (need 0 or 1)", z_format);
    if (bad_sizes(B, Tq, entry_stride)) return fail(CSA2_ERR_SHAPE, "sparse_attn: B=%d Tq=%d stride=%lld", B, Tq, (long long)entry_stride);
    if (H < 16 || H > 64 || H % 16) return fail(CSA2_ERR_UNSUPPORTED, "sparse_attn: H=%d (need 16, 32, 48 or 64)", H);
    if (Tq == 0) return ok();     // no work: no pointer is read
    if (!q_pos0 || !Q || !w_codes || !w_scale || !z_codes || !z_scales || !idx || !cnt || !sink ||
        !rope_cos || !rope_sin || !O)
        return fail(CSA2_ERR_NULL, "sparse_attn: a required pointer is NULL");
    if ((int64_t)cap < (int64_t)Tq + WINDOW - 1)
        return fail(CSA2_ERR_RANGE, "sparse_attn: window ring cap=%d < Tq+127=%lld", cap, (long long)Tq + WINDOW - 1);
    if (rope_rows < 1) return fail(CSA2_ERR_RANGE, "sparse_attn: empty rotary table");
    const size_t need = attn_ws(B, Tq, H, entry_stride).total;
    if (Tq > 0 && need > 0 && (!ws || ws_bytes < need))
        return fail(CSA2_ERR_WORKSPACE, "sparse_attn: workspace %zu < %zu bytes", ws_bytes, need);
    csa2_status s = launch_attn(B, Tq, H, q_pos0, Q, w_codes, w_scale, cap, z_codes, z_scales,
                                entry_stride, z_format, idx, cnt, sink, rope_cos, rope_sin,
                                rope_rows, O, lse, win_floor, ws, S(stream));
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_forward(int B, int T, int H, const int32_t* pos0, const uint16_t* kc,
                         const uint16_t* gc, const uint16_t* wn, const float* gamma_c,
                         const uint16_t* w_ik, const float* gamma_ik, const uint16_t* ki_given,
                         const uint16_t* Q, const uint16_t* qI, const float* wI, const float* sink,
                         const float* rope_cos, const float* rope_sin, int64_t rope_rows,
                         uint8_t* z_codes, uint8_t* z_scales, uint8_t* ki_codes,
                         uint8_t* ki_scales, int64_t entry_stride, int ratio, int z_format,
                         const int32_t* n_entries, uint8_t* w_codes, float* w_scale, int cap,
                         int32_t* idx, int32_t* cnt, uint16_t* O, float* lse,
                         const int32_t* win_floor, void* ws, size_t ws_bytes, void* stream) {
    if (bad_sizes(B, T, entry_stride)) return fail(CSA2_ERR_SHAPE, "forward: B=%d T=%d stride=%lld", B, T, (long long)entry_stride);
    if (bad_ratio(ratio)) return fail(CSA2_ERR_UNSUPPORTED, "forward: ratio=%d (need 1 or 2)", ratio);
    if (bad_zfmt(z_format)) return fail(CSA2_ERR_UNSUPPORTED, "forward: z_format=%d (need 0 or 1)", z_format);
    const int rsh = ratio == 2 ? 1 : 0;
    if (H < 16 || H > 64 || H % 16) return fail(CSA2_ERR_UNSUPPORTED, "forward: H=%d (need 16, 32, 48 or 64)", H);
    const bool prefill = kc != nullptr;
    if (T == 0) return ok();     // no work: no pointer is read
    if (!pos0 || !Q || !qI || !wI || !sink || !rope_cos || !rope_sin || !z_codes || !z_scales ||
        !ki_codes || !ki_scales || !w_codes || !w_scale || !idx || !cnt || !O)
        return fail(CSA2_ERR_NULL, "forward: a required pointer is NULL");
    if (prefill && ((ratio == 2 && !gc) || !wn || !gamma_c || (w_ik ? !gamma_ik : !ki_given)))
        return fail(CSA2_ERR_NULL, "forward: prefill needs gc (ratio 2), wn, gamma_c and w_ik+gamma_ik or ki_given");
    if (!prefill && !n_entries) return fail(CSA2_ERR_NULL, "forward: decode needs n_entries");
    if ((int64_t)cap < (int64_t)T + WINDOW - 1)
        return fail(CSA2_ERR_RANGE, "forward: window ring cap=%d < T+127=%lld", cap, (long long)T + WINDOW - 1);
    if (rope_rows < 1) return fail(CSA2_ERR_RANGE, "forward: empty rotary table");
    const size_t need = csa2_workspace_size(CSA2_OP_FORWARD, B, T, H, entry_stride);
    if (!ws || ws_bytes < need)
        return fail(CSA2_ERR_WORKSPACE, "forward: workspace %zu < %zu bytes", ws_bytes, need);
    if (T == 0) return ok();
    hipStream_t st = S(stream);
    const size_t ne_off = need - align256((size_t)B * sizeof(int32_t));
    int32_t* ne = (int32_t*)((uint8_t*)ws + ne_off);
    if (wn) {
        hipLaunchKernelGGL(k_window_encode, dim3((unsigned)cdiv((int64_t)B * T, 4)), dim3(256), 0,
                           st, B, T, pos0, wn, rope_cos, rope_sin, rope_rows, w_codes, w_scale,
                           cap);
    }
    if (prefill) {
        const int64_t items = (int64_t)B * (T >> rsh);
        if (items > 0)
            hipLaunchKernelGGL(k_compress, dim3((unsigned)cdiv(items, 4)), dim3(256), 0, st, B, T,
                               pos0, kc, gc, gamma_c, w_ik, gamma_ik, ki_given, rope_cos,
                               rope_sin, rope_rows, z_codes, z_scales, ki_codes, ki_scales,
                               entry_stride, rsh, z_format);
        if (!n_entries) {
            hipLaunchKernelGGL(k_prefill_entries, dim3((unsigned)cdiv(B, 256)), dim3(256), 0, st,
                               B, T, pos0, entry_stride, ne, rsh);
            n_entries = ne;
        }
    }
    csa2_status s = check_launch("csa2_forward (encode)");
    if (s != CSA2_OK) return s;
    s = launch_index(B, T, pos0, n_entries, qI, wI, ki_codes, ki_scales, entry_stride, rsh, idx,
                     cnt, ws, st);
    if (s != CSA2_OK) return s;
    s = launch_attn(B, T, H, pos0, Q, w_codes, w_scale, cap, z_codes, z_scales, entry_stride,
                    z_format, idx, cnt, sink, rope_cos, rope_sin, rope_rows, O, lse, win_floor,
                    ws, st);
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_quant_index_query(const uint16_t* qI, const float* wI, int64_t rows, uint8_t* q8,
                                   float* wq, void* stream) {
    if (rows < 0) return fail(CSA2_ERR_SHAPE, "quant_index_query: rows=%lld", (long long)rows);
    if (rows == 0) return ok();     // no work: no pointer is read
    if (!qI || !wI || !q8 || !wq) return fail(CSA2_ERR_NULL, "quant_index_query: NULL pointer");
    hipLaunchKernelGGL(k_quant_index_query, dim3((unsigned)cdiv(rows, 16)), dim3(256), 0,
                       S(stream), qI, wI, rows, q8, wq);
    csa2_status s = check_launch("csa2_quant_index_query");
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_encode_fp4_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes,
                                 uint8_t* scales, void* stream) {
    if (rows < 0 || cols < 32 || cols % 32) return fail(CSA2_ERR_SHAPE, "encode_fp4_rows: rows=%lld cols=%d", (long long)rows, cols);
    if (rows == 0) return ok();     // no work: no pointer is read
    if (!x || !codes || !scales) return fail(CSA2_ERR_NULL, "encode_fp4_rows: NULL pointer");
    const int64_t items = rows * (cols / 32);
    if (items == 0) return ok();
    hipLaunchKernelGGL(k_encode_fp4_rows, dim3((unsigned)cdiv(items, 256)), dim3(256), 0,
                       S(stream), x, rows, cols, codes, scales);
    csa2_status s = check_launch("csa2_encode_fp4_rows");
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_encode_fp4e4_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes,
                                   uint8_t* scales, void* stream) {
    if (rows < 0 || cols < 16 || cols % 16) return fail(CSA2_ERR_SHAPE, "encode_fp4e4_rows: rows=%lld cols=%d", (long long)rows, cols);
    if (rows == 0) return ok();     // no work: no pointer is read
    if (!x || !codes || !scales) return fail(CSA2_ERR_NULL, "encode_fp4e4_rows: NULL pointer");
    const int64_t items = rows * (cols / 16);
    if (items == 0) return ok();
    hipLaunchKernelGGL(k_encode_fp4e4_rows, dim3((unsigned)cdiv(items, 256)), dim3(256), 0,
                       S(stream), x, rows, cols, codes, scales);
    csa2_status s = check_launch("csa2_encode_fp4e4_rows");
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_decode_fp4e4_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                   int cols, uint16_t* out, void* stream) {
    if (rows < 0 || cols < 16 || cols % 16) return fail(CSA2_ERR_SHAPE, "decode_fp4e4_rows: rows=%lld cols=%d", (long long)rows, cols);
    if (rows == 0) return ok();     // no work: no pointer is read
    if (!codes || !scales || !out) return fail(CSA2_ERR_NULL, "decode_fp4e4_rows: NULL pointer");
    const int64_t items = rows * (cols / 8);
    if (items == 0) return ok();
    hipLaunchKernelGGL(k_decode_fp4e4_rows, dim3((unsigned)cdiv(items, 256)), dim3(256), 0,
                       S(stream), codes, scales, rows, cols, out);
    csa2_status s = check_launch("csa2_decode_fp4e4_rows");
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_encode_fp8_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes,
                                 float* scale, void* stream) {
    if (rows < 0 || cols < 1 || cols > 1024) return fail(CSA2_ERR_SHAPE, "encode_fp8_rows: rows=%lld cols=%d", (long long)rows, cols);
    if (rows == 0) return ok();     // no work: no pointer is read
    if (!x || !codes || !scale) return fail(CSA2_ERR_NULL, "encode_fp8_rows: NULL pointer");
    if (rows == 0) return ok();
    hipLaunchKernelGGL(k_encode_fp8_rows, dim3((unsigned)cdiv(rows, 4)), dim3(256), 0, S(stream),
                       x, rows, cols, codes, scale);
    csa2_status s = check_launch("csa2_encode_fp8_rows");
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_decode_fp4_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                 int cols, uint16_t* out, void* stream) {
    if (rows < 0 || cols < 32 || cols % 32) return fail(CSA2_ERR_SHAPE, "decode_fp4_rows: rows=%lld cols=%d", (long long)rows, cols);
    if (rows == 0) return ok();     // no work: no pointer is read
    if (!codes || !scales || !out) return fail(CSA2_ERR_NULL, "decode_fp4_rows: NULL pointer");
    const int64_t items = rows * (cols / 8);
    if (items == 0) return ok();
    hipLaunchKernelGGL(k_decode_fp4_rows, dim3((unsigned)cdiv(items, 256)), dim3(256), 0,
                       S(stream), codes, scales, rows, cols, out);
    csa2_status s = check_launch("csa2_decode_fp4_rows");
    return s == CSA2_OK ? ok() : s;
}

csa2_status csa2_decode_fp8_rows(const uint8_t* codes, int64_t rows, int cols, uint16_t* out,
                                 void* stream) {
    if (rows < 0 || cols < 8 || cols % 8) return fail(CSA2_ERR_SHAPE, "decode_fp8_rows: rows=%lld cols=%d", (long long)rows, cols);
    if (rows == 0) return ok();     // no work: no pointer is read
    if (!codes || !out) return fail(CSA2_ERR_NULL, "decode_fp8_rows: NULL pointer");
    const int64_t items = rows * (cols / 8);
    if (items == 0) return ok();
    hipLaunchKernelGGL(k_decode_fp8_rows, dim3((unsigned)cdiv(items, 256)), dim3(256), 0,
                       S(stream), codes, rows, cols, out);
    csa2_status s = check_launch("csa2_decode_fp8_rows");
    return s == CSA2_OK ? ok() : s;
}

}  // extern "C"
