// noalloc.hip -- paged_attn_decode_static(): phase 1 and phase 2 of the
// decode in one call, for callers that cannot allocate device memory. The
// split partials that paged_attn_decode() takes as caller workspaces live in
// `scratch`, a file-scope device array of PA_STATIC_SCRATCH_BYTES that every
// GPU the library runs on holds until the process ends.
//
// `scratch` names a host-side stand-in in host code, not a device address.
// Its address on a device comes from hipGetSymbolAddress, taken once per
// device (with that device current) on the first call there, and is the only
// form host code ever passes on.
#include <stdio.h>

#include <mutex>
#include <string>

#include "kernels.h"

#define PA_EXPORT extern "C" __attribute__((visibility("default")))

static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device

int fail_static(int code, const char* msg)
{
    char buf[512];
    snprintf(buf, sizeof buf, "paged_attn_decode_static: %s", msg);
    pa::set_last_error(buf);
    return code;
}

// Device address of `scratch` on `dev`, looked up once per device with that
// device current.
int scratch_on(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices) return PA_ENOTSUP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return PA_ELAUNCH;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return PA_ELAUNCH;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) return PA_ELAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace

PA_EXPORT int paged_attn_decode_static(const pa_decode_args* a, void* output, int64_t out_stride_s,
                                       int64_t out_stride_h, int32_t out_dtype, void* stream)
{
    if (!a) return fail_static(PA_EINVAL, "args is NULL");
    if (a->tmp_output || a->exp_sums || a->max_logits)
        return fail_static(PA_EINVAL, "tmp_output, exp_sums and max_logits must be NULL (the library's scratch "
                                      "buffer holds the partials)");
    if (a->num_seqs < 0 || a->num_heads < 1 || a->v_head_size < 1 || a->max_num_parts < 1 || a->num_group < 0)
        return fail_static(PA_EINVAL, "num_seqs, num_group >= 0 and num_heads, v_head_size, max_num_parts >= 1 "
                                      "required");
    if (a->tmp_dtype != PA_F32 && a->tmp_dtype != PA_F16 && a->tmp_dtype != PA_BF16)
        return fail_static(PA_EINVAL, "tmp_dtype is not PA_F32, PA_F16 or PA_BF16");
    const int64_t esz = a->tmp_dtype == PA_F32 ? 4 : 2;  // bytes per partial value
    const int64_t rows = (int64_t)a->num_seqs * (a->num_group < 1 ? 1 : a->num_group);
    const int64_t slots = rows * a->num_heads * a->max_num_parts;  // (row, head, split) triples
    const int64_t bytes = slots * ((int64_t)a->v_head_size * esz + 8);
    if (bytes > (int64_t)PA_STATIC_SCRATCH_BYTES) {
        char buf[256];
        snprintf(buf, sizeof buf,
                 "the partials need %lld bytes (rows %lld x heads %d x splits %d x (v_head_size %d x %d + 8)), "
                 "more than the %lld-byte scratch buffer",
                 (long long)bytes, (long long)rows, a->num_heads, a->max_num_parts, a->v_head_size, (int)esz,
                 (long long)PA_STATIC_SCRATCH_BYTES);
        return fail_static(PA_EINVAL, buf);
    }
    if (rows == 0) return PA_OK;
    if (!output) return fail_static(PA_EINVAL, "output is NULL");

    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev) != hipSuccess)
            return fail_static(PA_EINVAL, "cannot query the stream's device");
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return fail_static(PA_ELAUNCH, "no current device");
    }
    void* base = nullptr;
    const int rc = scratch_on(dev, &base);
    if (rc != PA_OK) return fail_static(rc, "cannot look up the scratch buffer on the stream's device");

    // partials, contiguous: tmp [rows, H, P, Dv] of tmp_dtype, then max_logits
    // and exp_sums [rows, H, P] (every supported v_head_size is a multiple
    // of 64, so both start 128-byte aligned; others are rejected by phase 1)
    char* tmp = static_cast<char*>(base);
    float* ml = reinterpret_cast<float*>(tmp + slots * a->v_head_size * esz);
    float* es = ml + slots;
    pa_decode_args d = *a;
    d.tmp_output = tmp;
    d.tmp_stride_d = 1;
    d.tmp_stride_p = a->v_head_size;
    d.tmp_stride_h = (int64_t)a->max_num_parts * a->v_head_size;
    d.tmp_stride_s = (int64_t)a->num_heads * d.tmp_stride_h;
    d.max_logits = ml;
    d.exp_sums = es;
    d.ml_stride_p = 1;
    d.ml_stride_h = a->max_num_parts;
    d.ml_stride_s = (int64_t)a->num_heads * a->max_num_parts;
    int r = paged_attn_decode(&d, stream);
    if (r != PA_OK) return fail_static(r, pa_last_error());
    pa_reduce_args q{};
    q.output = output;
    q.out_stride_s = out_stride_s;
    q.out_stride_h = out_stride_h;
    q.out_stride_d = 1;
    q.out_dtype = out_dtype;
    q.tmp_output = tmp;
    q.tmp_stride_s = d.tmp_stride_s;
    q.tmp_stride_h = d.tmp_stride_h;
    q.tmp_stride_p = d.tmp_stride_p;
    q.tmp_stride_d = 1;
    q.exp_sums = es;
    q.max_logits = ml;
    q.ml_stride_s = d.ml_stride_s;
    q.ml_stride_h = d.ml_stride_h;
    q.ml_stride_p = 1;
    q.seq_lens = a->seq_lens;
    q.num_splits = a->num_splits;
    q.num_seqs = a->num_seqs;
    q.num_heads = a->num_heads;
    q.v_head_size = a->v_head_size;
    q.partition_size = a->partition_size;
    q.max_num_parts = a->max_num_parts;
    q.num_group = a->num_group;
    q.tmp_dtype = a->tmp_dtype;
    r = paged_attn_reduce(&q, stream);
    return r == PA_OK ? r : fail_static(r, pa_last_error());
}
