/* CPython binding of the per-call entry points (lora_apply, lora_apply_ranked,
 * lora_apply_device): argument marshalling only.  A serving loop calls one of
 * these once per layer and step; through ctypes the conversion of their 14 to
 * 16 arguments costs more host time than the library's own plan for a small
 * decode batch, and the host then paces the GPU.  Here each argument is one
 * integer conversion.
 *
 * The library is the one ctypes has loaded: every call takes the entry
 * point's address (ctypes.cast(lib.lora_apply, c_void_p).value) as its first
 * argument and calls through a pointer of the entry point's own type, so this
 * module links nothing and cannot bind a second copy of the library.  Pointer
 * arguments are Python ints (None is NULL); the return value is the entry
 * point's status.  The GIL is released around the call, as ctypes does. */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stdint.h>

#include "lora_pool.h"

typedef int32_t (*apply_fn)(const lora_pool_desc*, const void*, const void*, const void*, void*,
                            int32_t, const int32_t*, const uint8_t*, int32_t, void*, int64_t,
                            void*, int64_t, void*);
typedef int32_t (*apply_ranked_fn)(const lora_pool_desc*, const void*, const void*, const void*,
                                   void*, int32_t, const int32_t*, const uint8_t*, int32_t,
                                   const int32_t*, void*, int64_t, void*, int64_t, void*);
typedef int32_t (*apply_device_fn)(const lora_pool_desc*, const void*, const void*, const void*,
                                   void*, int32_t, const int32_t*, const uint8_t*, int32_t, void*,
                                   int64_t, void*);

/* the typedefs match the header's declarations */
_Static_assert(__builtin_types_compatible_p(__typeof__(&lora_apply), apply_fn), "lora_apply");
_Static_assert(__builtin_types_compatible_p(__typeof__(&lora_apply_ranked), apply_ranked_fn),
               "lora_apply_ranked");
_Static_assert(__builtin_types_compatible_p(__typeof__(&lora_apply_device), apply_device_fn),
               "lora_apply_device");

/* kinds of argument */
enum { P = 0, I32 = 1, I64 = 2 };

/* Converts args[0 .. n) by kind into out[]; returns 0, or -1 with a Python
 * exception set. */
static int convert(PyObject* const* args, Py_ssize_t nargs, const char* name, const int* kinds,
                   int n, uint64_t* out) {
  if (nargs != n) {
    PyErr_Format(PyExc_TypeError, "%s takes %d arguments (%zd given)", name, n, nargs);
    return -1;
  }
  for (int i = 0; i < n; ++i) {
    PyObject* a = args[i];
    if (kinds[i] == P) {
      if (a == Py_None) {
        out[i] = 0;
        continue;
      }
      const unsigned long long v = PyLong_AsUnsignedLongLong(a);
      if (v == (unsigned long long)-1 && PyErr_Occurred()) return -1;
      out[i] = v;
    } else {
      const long long v = PyLong_AsLongLong(a);
      if (v == -1 && PyErr_Occurred()) return -1;
      if (kinds[i] == I32 && (v < INT32_MIN || v > INT32_MAX)) {
        PyErr_Format(PyExc_OverflowError, "%s: argument %d does not fit int32", name, i);
        return -1;
      }
      out[i] = (uint64_t)v;
    }
  }
  if (out[0] == 0) {
    PyErr_Format(PyExc_ValueError, "%s: NULL entry point address", name);
    return -1;
  }
  return 0;
}

#define PTR(i) ((void*)(uintptr_t)a[i])
#define I32V(i) ((int32_t)(int64_t)a[i])
#define I64V(i) ((int64_t)a[i])

/* apply(fn, desc, A_pool, B_pool, x, y, T, ids_host, prefill_host,
 *       bgmv_max_rank, ws, ws_bytes, meta_host, meta_host_bytes, stream) */
static PyObject* py_apply(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
  (void)self;
  static const int kinds[15] = {P, P, P, P, P, P, I32, P, P, I32, P, I64, P, I64, P};
  uint64_t a[15];
  if (convert(args, nargs, "apply", kinds, 15, a)) return NULL;
  const apply_fn f = (apply_fn)(uintptr_t)a[0];
  int32_t st;
  Py_BEGIN_ALLOW_THREADS
  st = f((const lora_pool_desc*)PTR(1), PTR(2), PTR(3), PTR(4), PTR(5), I32V(6),
         (const int32_t*)PTR(7), (const uint8_t*)PTR(8), I32V(9), PTR(10), I64V(11), PTR(12),
         I64V(13), PTR(14));
  Py_END_ALLOW_THREADS
  return PyLong_FromLong(st);
}

/* apply_ranked(fn, desc, A_pool, B_pool, x, y, T, ids_host, prefill_host,
 *              bgmv_max_rank, slot_ranks, ws, ws_bytes, meta_host,
 *              meta_host_bytes, stream) */
static PyObject* py_apply_ranked(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
  (void)self;
  static const int kinds[16] = {P, P, P, P, P, P, I32, P, P, I32, P, P, I64, P, I64, P};
  uint64_t a[16];
  if (convert(args, nargs, "apply_ranked", kinds, 16, a)) return NULL;
  const apply_ranked_fn f = (apply_ranked_fn)(uintptr_t)a[0];
  int32_t st;
  Py_BEGIN_ALLOW_THREADS
  st = f((const lora_pool_desc*)PTR(1), PTR(2), PTR(3), PTR(4), PTR(5), I32V(6),
         (const int32_t*)PTR(7), (const uint8_t*)PTR(8), I32V(9), (const int32_t*)PTR(10),
         PTR(11), I64V(12), PTR(13), I64V(14), PTR(15));
  Py_END_ALLOW_THREADS
  return PyLong_FromLong(st);
}

/* apply_device(fn, desc, A_pool, B_pool, x, y, T, ids, prefill,
 *              bgmv_max_rank, ws, ws_bytes, stream) */
static PyObject* py_apply_device(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
  (void)self;
  static const int kinds[13] = {P, P, P, P, P, P, I32, P, P, I32, P, I64, P};
  uint64_t a[13];
  if (convert(args, nargs, "apply_device", kinds, 13, a)) return NULL;
  const apply_device_fn f = (apply_device_fn)(uintptr_t)a[0];
  int32_t st;
  Py_BEGIN_ALLOW_THREADS
  st = f((const lora_pool_desc*)PTR(1), PTR(2), PTR(3), PTR(4), PTR(5), I32V(6),
         (const int32_t*)PTR(7), (const uint8_t*)PTR(8), I32V(9), PTR(10), I64V(11), PTR(12));
  Py_END_ALLOW_THREADS
  return PyLong_FromLong(st);
}

static PyMethodDef methods[] = {
    {"apply", (PyCFunction)(void (*)(void))py_apply, METH_FASTCALL,
     "apply(fn, desc, A_pool, B_pool, x, y, T, ids_host, prefill_host, bgmv_max_rank, ws, "
     "ws_bytes, meta_host, meta_host_bytes, stream) -> status of lora_apply"},
    {"apply_ranked", (PyCFunction)(void (*)(void))py_apply_ranked, METH_FASTCALL,
     "apply_ranked(fn, desc, A_pool, B_pool, x, y, T, ids_host, prefill_host, bgmv_max_rank, "
     "slot_ranks, ws, ws_bytes, meta_host, meta_host_bytes, stream) -> status of "
     "lora_apply_ranked"},
    {"apply_device", (PyCFunction)(void (*)(void))py_apply_device, METH_FASTCALL,
     "apply_device(fn, desc, A_pool, B_pool, x, y, T, ids, prefill, bgmv_max_rank, ws, "
     "ws_bytes, stream) -> status of lora_apply_device"},
    {NULL, NULL, 0, NULL}};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_lora_call",
                                    "CPython binding of the per-call entry points", -1, methods,
                                    NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__lora_call(void) { return PyModule_Create(&module); }
