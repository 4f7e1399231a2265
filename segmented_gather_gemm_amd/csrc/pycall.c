/*
 * CPython entry points for the hot calls of libsgg_lora: argument
 * marshalling only.  Each function has the name of the C entry point it
 * calls, takes that entry point's arguments in order as Python integers
 * (device and host addresses as ints, 0 or None for NULL) and returns its
 * status.  Converting integers here costs a fraction of a microsecond per
 * call, against several microseconds for a ctypes call with twenty-odd
 * arguments, which matters for a decode step of a few tens of microseconds.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stdint.h>
#include <string.h>

#include "sgg_lora.h"

/* Host buffers exported by the arguments of one call (NumPy arrays passed
 * for host pointers), held until the call returns. */
#define MAX_HELD 8
typedef struct {
  Py_buffer view[MAX_HELD];
  int n;
} Held;

static void release(Held* held) {
  for (int i = 0; i < held->n; ++i) PyBuffer_Release(&held->view[i]);
  held->n = 0;
}

/* Convert args[i] by sig[i]: 'p' pointer -- an integer address, None (NULL)
 * or a C-contiguous buffer (its first byte, e.g. a NumPy array's data);
 * 'l' int64; 'i' int32. */
static int convert(const char* name, const char* sig, PyObject* const* args, Py_ssize_t nargs,
                   int64_t* out, Held* held) {
  const Py_ssize_t want = (Py_ssize_t)strlen(sig);
  held->n = 0;
  if (nargs != want) {
    PyErr_Format(PyExc_TypeError, "%s takes %zd arguments (%zd given)", name, want, nargs);
    return 0;
  }
  for (Py_ssize_t k = 0; k < want; ++k) {
    PyObject* a = args[k];
    if (sig[k] == 'p') {
      if (a == Py_None) {
        out[k] = 0;
        continue;
      }
      if (!PyLong_Check(a) && PyObject_CheckBuffer(a)) {
        if (held->n == MAX_HELD) {
          PyErr_Format(PyExc_TypeError, "%s: too many buffer arguments", name);
          release(held);
          return 0;
        }
        if (PyObject_GetBuffer(a, &held->view[held->n], PyBUF_C_CONTIGUOUS) < 0) {
          release(held);
          return 0;
        }
        out[k] = (int64_t)(uintptr_t)held->view[held->n].buf;
        ++held->n;
        continue;
      }
      unsigned long long v;
      if (PyLong_CheckExact(a)) {
        v = PyLong_AsUnsignedLongLong(a);
      } else {  /* integer-like objects (NumPy scalars) */
        PyObject* idx = PyNumber_Index(a);
        if (idx == NULL) goto bad;
        v = PyLong_AsUnsignedLongLong(idx);
        Py_DECREF(idx);
      }
      if (v == (unsigned long long)-1 && PyErr_Occurred()) goto bad;
      out[k] = (int64_t)v;
    } else {
      const long long v = PyLong_AsLongLong(a);
      if (v == -1 && PyErr_Occurred()) goto bad;
      if (sig[k] == 'i' && (v < INT32_MIN || v > INT32_MAX)) {
        PyErr_Format(PyExc_OverflowError, "%s: argument %zd does not fit in int32", name, k);
        release(held);
        return 0;
      }
      out[k] = (int64_t)v;
    }
    continue;
  bad:
    PyErr_Clear();
    PyErr_Format(PyExc_TypeError, "%s: argument %zd must be an integer%s", name, k,
                 sig[k] == 'p' ? " address, a contiguous buffer or None" : "");
    release(held);
    return 0;
  }
  return 1;
}

/* Argument signature of each entry point, in the order of its C parameters:
 * 'p' pointer, 'l' int64_t, 'i' int32_t.  Also exported as the module's
 * SIGNATURES dict. */
#define SIG_lora_plan_max_segments "lii"
#define SIG_lora_plan_upload "ppippiiiiliipplppip"
#define SIG_lora_plan_upload_embedding "ppippiiiiliipplppipplplilp"
#define SIG_lora_plan_lm_head_upload "ppippiiiliipplppip"
#define SIG_lora_plan_device "ppippiiiiliiplpp"
#define SIG_lora_shrink_workspace_bytes "lliiii"
#define SIG_lora_qkv_workspace_bytes "lliiii"
#define SIG_lora_shrink "plppllliiippippiplp"
#define SIG_lora_expand "plplplliipiippipppip"
#define SIG_lora_qkv "plpplpllliipiippipppiplp"
#define SIG_lora_a_embedding "pplplliilppippip"

/* One int64 per argument, sized by the signature string; CALL runs the
 * entry point, then releases the held buffers. */
#define CONVERT(fn)                   \
  int64_t v[sizeof(SIG_##fn) - 1];    \
  Held held;                          \
  if (!convert(#fn, SIG_##fn, args, n, v, &held)) return NULL
#define RETURN_INT(expr)              \
  do {                                \
    const long long rc_ = (expr);     \
    release(&held);                   \
    return PyLong_FromLongLong(rc_);  \
  } while (0)

#define P(k) ((void*)(uintptr_t)v[k])
#define I32P(k) ((int32_t*)(uintptr_t)v[k])
#define L(k) (v[k])
#define I(k) ((int32_t)v[k])

static PyObject* py_lora_plan_max_segments(PyObject* self, PyObject* const* args, Py_ssize_t n) {
  CONVERT(lora_plan_max_segments);
  RETURN_INT(lora_plan_max_segments(L(0), I(1), I(2)));
}

static PyObject* py_lora_plan_upload(PyObject* self, PyObject* const* args, Py_ssize_t n) {
  CONVERT(lora_plan_upload);
  RETURN_INT(lora_plan_upload(
      I32P(0), I32P(1), I(2), I32P(3), (const float*)P(4), I(5), I(6), I(7), I(8), L(9), I(10),
      I(11), P(12), P(13), L(14), I32P(15), I32P(16), I(17), P(18)));
}

static PyObject* py_lora_plan_upload_embedding(PyObject* self, PyObject* const* args,
                                               Py_ssize_t n) {
  CONVERT(lora_plan_upload_embedding);
  RETURN_INT(lora_plan_upload_embedding(
      I32P(0), I32P(1), I(2), I32P(3), (const float*)P(4), I(5), I(6), I(7), I(8), L(9), I(10),
      I(11), P(12), P(13), L(14), I32P(15), I32P(16), I(17), (const int64_t*)P(18), P(19),
      L(20), P(21), L(22), I(23), L(24), P(25)));
}

static PyObject* py_lora_plan_device(PyObject* self, PyObject* const* args, Py_ssize_t n) {
  CONVERT(lora_plan_device);
  RETURN_INT(lora_plan_device(I32P(0), I32P(1), I(2), I32P(3), (const float*)P(4), I(5), I(6),
                              I(7), I(8), L(9), I(10), I(11), P(12), L(13), I32P(14), P(15)));
}

static PyObject* py_lora_plan_lm_head_upload(PyObject* self, PyObject* const* args,
                                             Py_ssize_t n) {
  CONVERT(lora_plan_lm_head_upload);
  RETURN_INT(lora_plan_lm_head_upload(
      I32P(0), I32P(1), I(2), I32P(3), (const float*)P(4), I(5), I(6), I(7), L(8), I(9), I(10),
      P(11), P(12), L(13), I32P(14), I32P(15), I(16), P(17)));
}

static PyObject* py_lora_shrink_workspace_bytes(PyObject* self, PyObject* const* args,
                                                Py_ssize_t n) {
  CONVERT(lora_shrink_workspace_bytes);
  RETURN_INT(lora_shrink_workspace_bytes(L(0), L(1), I(2), I(3), I(4), I(5)));
}

static PyObject* py_lora_qkv_workspace_bytes(PyObject* self, PyObject* const* args,
                                             Py_ssize_t n) {
  CONVERT(lora_qkv_workspace_bytes);
  RETURN_INT(lora_qkv_workspace_bytes(L(0), L(1), I(2), I(3), I(4), I(5)));
}

static PyObject* py_lora_shrink(PyObject* self, PyObject* const* args, Py_ssize_t n) {
  CONVERT(lora_shrink);
  RETURN_INT(lora_shrink(P(0), L(1), P(2), P(3), L(4), L(5), L(6), I(7), I(8), I(9),
                                     I32P(10), I32P(11), I(12), I32P(13), I32P(14), I(15), P(16),
                                     L(17), P(18)));
}

static PyObject* py_lora_expand(PyObject* self, PyObject* const* args, Py_ssize_t n) {
  CONVERT(lora_expand);
  RETURN_INT(lora_expand(P(0), L(1), P(2), L(3), P(4), L(5), L(6), I(7), I(8),
                                     I32P(9), I(10), I(11), I32P(12), I32P(13), I(14), I32P(15),
                                     I32P(16), (const float*)P(17), I(18), P(19)));
}

static PyObject* py_lora_qkv(PyObject* self, PyObject* const* args, Py_ssize_t n) {
  CONVERT(lora_qkv);
  RETURN_INT(lora_qkv(P(0), L(1), P(2), P(3), L(4), P(5), L(6), L(7), L(8), I(9),
                                  I(10), I32P(11), I(12), I(13), I32P(14), I32P(15), I(16),
                                  I32P(17), I32P(18), (const float*)P(19), I(20), P(21), L(22),
                                  P(23)));
}

static PyObject* py_lora_a_embedding(PyObject* self, PyObject* const* args, Py_ssize_t n) {
  CONVERT(lora_a_embedding);
  RETURN_INT(lora_a_embedding((const int64_t*)P(0), P(1), L(2), P(3), L(4), L(5),
                                          I(6), I(7), L(8), I32P(9), I32P(10), I(11), I32P(12),
                                          I32P(13), I(14), P(15)));
}

#define ENTRY(fn) {#fn, (PyCFunction)(void (*)(void))py_##fn, METH_FASTCALL, NULL}

static PyMethodDef methods[] = {
    ENTRY(lora_plan_max_segments),
    ENTRY(lora_plan_upload),
    ENTRY(lora_plan_upload_embedding),
    ENTRY(lora_plan_lm_head_upload),
    ENTRY(lora_plan_device),
    ENTRY(lora_shrink_workspace_bytes),
    ENTRY(lora_qkv_workspace_bytes),
    ENTRY(lora_shrink),
    ENTRY(lora_expand),
    ENTRY(lora_qkv),
    ENTRY(lora_a_embedding),
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef module = {
    PyModuleDef_HEAD_INIT, "_sggcall",
    "Hot calls of libsgg_lora with integer arguments (marshalling only).", -1, methods,
};

PyMODINIT_FUNC PyInit__sggcall(void) {
  PyObject* m = PyModule_Create(&module);
  if (m == NULL) return NULL;
  PyObject* sigs = Py_BuildValue(
      "{ssssssssssssssssssssss}", "lora_plan_max_segments", SIG_lora_plan_max_segments,
      "lora_plan_device", SIG_lora_plan_device, "lora_plan_upload_embedding",
      SIG_lora_plan_upload_embedding,
      "lora_plan_upload", SIG_lora_plan_upload, "lora_plan_lm_head_upload",
      SIG_lora_plan_lm_head_upload, "lora_shrink_workspace_bytes",
      SIG_lora_shrink_workspace_bytes, "lora_qkv_workspace_bytes", SIG_lora_qkv_workspace_bytes,
      "lora_shrink", SIG_lora_shrink, "lora_expand", SIG_lora_expand, "lora_qkv", SIG_lora_qkv,
      "lora_a_embedding", SIG_lora_a_embedding);
  if (sigs == NULL || PyModule_AddObject(m, "SIGNATURES", sigs) < 0) {
    Py_XDECREF(sigs);
    Py_DECREF(m);
    return NULL;
  }
  return m;
}
