// Tensor-descriptor entry points (pa_reshape_and_cache_t, pa_decode_t):
// host-side checks that the arrays agree with one another, then the flat
// calls. Plain C++: nothing here touches the device.
#include <cstdint>

#include "pa.h"
#include "pa_error.h"

namespace {

using pa::fail;

// A descriptor of the given rank with non-negative sizes whose element count
// fits 2^62; if it is not empty, dense row-major (a size-1 dimension may have
// any stride) and with data. An empty tensor's strides are not looked at.
int check_tensor(const pa_tensor* t, const char* call, const char* name, int ndim) {
  if (!t) return fail(PA_ERR_NULL, "%s: NULL descriptor for %s", call, name);
  if (t->ndim != ndim) return fail(PA_ERR_SHAPE, "%s: %s has %d dimensions, expected %d", call, name, t->ndim, ndim);
  int64_t elems = 1;
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0) return fail(PA_ERR_SHAPE, "%s: %s has a negative size", call, name);
    if (t->shape[i] > 0 && elems > (INT64_C(1) << 62) / t->shape[i])
      return fail(PA_ERR_SHAPE, "%s: %s has too many elements", call, name);
    elems *= t->shape[i];
  }
  if (elems == 0) return PA_OK;
  int64_t expect = 1;
  for (int i = ndim - 1; i >= 0; --i) {
    if (t->shape[i] != 1 && t->stride[i] != expect)
      return fail(PA_ERR_SHAPE, "%s: %s must be dense row-major (dimension %d has stride %lld, expected %lld)", call,
                  name, i, (long long)t->stride[i], (long long)expect);
    expect *= t->shape[i];
  }
  if (!t->data) return fail(PA_ERR_NULL, "%s: %s has no data", call, name);
  return PA_OK;
}

// Sizes that must agree between two descriptors.
int same(int64_t a, int64_t b, const char* call, const char* what) {
  if (a != b) return fail(PA_ERR_SHAPE, "%s: %s disagree (%lld and %lld)", call, what, (long long)a, (long long)b);
  return PA_OK;
}

bool fits_int(int64_t x) { return x >= 0 && x <= 0x7fffffffLL; }

}  // namespace

extern "C" {

int pa_reshape_and_cache_t(const pa_tensor* key, const pa_tensor* value, const pa_tensor* k_cache,
                           const pa_tensor* v_cache, const pa_tensor* slot_mapping, float k_scale, float v_scale,
                           void* stream) {
  const char* c = "reshape_and_cache";
  int rc;
  if ((rc = check_tensor(key, c, "key", 3)) || (rc = check_tensor(value, c, "value", 3)) ||
      (rc = check_tensor(k_cache, c, "k_cache", 4)) || (rc = check_tensor(v_cache, c, "v_cache", 4)) ||
      (rc = check_tensor(slot_mapping, c, "slot_mapping", 1)))
    return rc;
  for (int i = 0; i < 3; ++i)
    if ((rc = same(key->shape[i], value->shape[i], c, "key and value shapes"))) return rc;
  for (int i = 0; i < 4; ++i)
    if ((rc = same(k_cache->shape[i], v_cache->shape[i], c, "k_cache and v_cache shapes"))) return rc;
  if (key->dtype != value->dtype) return fail(PA_ERR_DTYPE, "%s: key and value dtypes differ", c);
  if (k_cache->dtype != v_cache->dtype) return fail(PA_ERR_DTYPE, "%s: k_cache and v_cache dtypes differ", c);
  if ((rc = same(key->shape[1], k_cache->shape[1], c, "key and cache KV heads")) ||
      (rc = same(key->shape[2], k_cache->shape[3], c, "key and cache head sizes")) ||
      (rc = same(key->shape[0], slot_mapping->shape[0], c, "tokens of key and slot_mapping")))
    return rc;
  if (slot_mapping->dtype != PA_DTYPE_I32 && slot_mapping->dtype != PA_DTYPE_I64)
    return fail(PA_ERR_DTYPE, "%s: slot_mapping must be I32 or I64", c);
  if (!fits_int(key->shape[1]) || !fits_int(key->shape[2]) || !fits_int(k_cache->shape[2]))
    return fail(PA_ERR_SHAPE, "%s: a size does not fit an int", c);
  return pa_reshape_and_cache(key->data, value->data, k_cache->data, v_cache->data, slot_mapping->data,
                              slot_mapping->dtype == PA_DTYPE_I64, key->shape[0], (int)key->shape[1],
                              (int)key->shape[2], k_cache->shape[0], (int)k_cache->shape[2], key->dtype,
                              k_cache->dtype, k_scale, v_scale, stream);
}

int pa_decode_t(const pa_tensor* out, const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                const pa_tensor* block_tables, const pa_tensor* context_lens, float scale, int num_kv_heads,
                int block_size, float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                void* stream) {
  const char* c = "decode";
  int rc;
  if ((rc = check_tensor(out, c, "out", 3)) || (rc = check_tensor(q, c, "q", 3)) ||
      (rc = check_tensor(k_cache, c, "k_cache", 4)) || (rc = check_tensor(v_cache, c, "v_cache", 4)) ||
      (rc = check_tensor(block_tables, c, "block_tables", 2)) ||
      (rc = check_tensor(context_lens, c, "context_lens", 1)))
    return rc;
  for (int i = 0; i < 3; ++i)
    if ((rc = same(out->shape[i], q->shape[i], c, "out and q shapes"))) return rc;
  for (int i = 0; i < 4; ++i)
    if ((rc = same(k_cache->shape[i], v_cache->shape[i], c, "k_cache and v_cache shapes"))) return rc;
  if (k_cache->dtype != v_cache->dtype) return fail(PA_ERR_DTYPE, "%s: k_cache and v_cache dtypes differ", c);
  if ((rc = same(k_cache->shape[1], num_kv_heads, c, "cache KV heads and num_kv_heads")) ||
      (rc = same(k_cache->shape[2], block_size, c, "cache block size and block_size")) ||
      (rc = same(k_cache->shape[3], q->shape[2], c, "cache and q head sizes")) ||
      (rc = same(block_tables->shape[0], q->shape[0], c, "sequences of q and block_tables")) ||
      (rc = same(context_lens->shape[0], q->shape[0], c, "sequences of q and context_lens")))
    return rc;
  if (block_tables->dtype != PA_DTYPE_I32 || context_lens->dtype != PA_DTYPE_I32)
    return fail(PA_ERR_DTYPE, "%s: block_tables and context_lens must be I32", c);
  if (!fits_int(q->shape[0]) || !fits_int(q->shape[1]) || !fits_int(q->shape[2]) ||
      !fits_int(block_tables->shape[1]))
    return fail(PA_ERR_SHAPE, "%s: a size does not fit an int", c);
  return pa_decode(out->data, q->data, k_cache->data, v_cache->data,
                   static_cast<const int32_t*>(block_tables->data), static_cast<const int32_t*>(context_lens->data),
                   scale, num_kv_heads, block_size, (int)q->shape[0], (int)q->shape[1], (int)q->shape[2],
                   (int)block_tables->shape[1], k_cache->shape[0], q->dtype, k_cache->dtype, out->dtype, k_scale,
                   v_scale, workspace, workspace_bytes, stream);
}

}  // extern "C"
