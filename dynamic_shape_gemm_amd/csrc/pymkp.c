/* Argument marshalling for the GEMM entry points of libmkp.so, as a CPython
 * extension: integers in, the C ABI's status code out.  It exists because a
 * ctypes call converts each of its 10-14 arguments through Python objects,
 * which for the smallest GEMMs costs as much host time as the launch itself.
 * Every argument is a Python int (device addresses included); the stream is
 * the raw stream handle (void *, 0 for the null stream).  Nothing here
 * computes: each function converts its arguments and calls the entry point
 * of the same name.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stdint.h>

#include "mkp.h"

static int get_i64(PyObject* o, int64_t* v) {
    long long x = PyLong_AsLongLong(o);
    if (x == -1 && PyErr_Occurred()) return -1;
    *v = (int64_t)x;
    return 0;
}

static int get_ptr(PyObject* o, void** p) {
    void* x = PyLong_AsVoidPtr(o);
    if (x == NULL && PyErr_Occurred()) return -1;
    *p = x;
    return 0;
}

static int check_nargs(Py_ssize_t n, Py_ssize_t want, const char* name) {
    if (n != want) {
        PyErr_Format(PyExc_TypeError, "%s takes %zd arguments (%zd given)", name, want, n);
        return -1;
    }
    return 0;
}

/* (M, N, K, A, lda, B, ldb, C, ldc, stream) */
typedef int (*gemm_fn)(int64_t, int64_t, int64_t, const void*, int64_t, const void*, int64_t, float*, int64_t,
                       void*);
/* (batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream) */
typedef int (*batched_fn)(int64_t, int64_t, int64_t, int64_t, const void*, int64_t, int64_t, const void*, int64_t,
                          int64_t, float*, int64_t, int64_t, void*);

static PyObject* call_gemm(gemm_fn fn, const char* name, PyObject* const* a, Py_ssize_t n) {
    if (check_nargs(n, 10, name)) return NULL;
    int64_t M, N, K, lda, ldb, ldc;
    void *A, *B, *C, *st;
    if (get_i64(a[0], &M) || get_i64(a[1], &N) || get_i64(a[2], &K) || get_ptr(a[3], &A) || get_i64(a[4], &lda) ||
        get_ptr(a[5], &B) || get_i64(a[6], &ldb) || get_ptr(a[7], &C) || get_i64(a[8], &ldc) || get_ptr(a[9], &st))
        return NULL;
    return PyLong_FromLong(fn(M, N, K, A, lda, B, ldb, (float*)C, ldc, st));
}

static PyObject* call_batched(batched_fn fn, const char* name, PyObject* const* a, Py_ssize_t n) {
    if (check_nargs(n, 14, name)) return NULL;
    int64_t bt, M, N, K, lda, sA, ldb, sB, ldc, sC;
    void *A, *B, *C, *st;
    if (get_i64(a[0], &bt) || get_i64(a[1], &M) || get_i64(a[2], &N) || get_i64(a[3], &K) || get_ptr(a[4], &A) ||
        get_i64(a[5], &lda) || get_i64(a[6], &sA) || get_ptr(a[7], &B) || get_i64(a[8], &ldb) ||
        get_i64(a[9], &sB) || get_ptr(a[10], &C) || get_i64(a[11], &ldc) || get_i64(a[12], &sC) ||
        get_ptr(a[13], &st))
        return NULL;
    return PyLong_FromLong(fn(bt, M, N, K, A, lda, sA, B, ldb, sB, (float*)C, ldc, sC, st));
}

static PyObject* py_gemm(PyObject* self, PyObject* const* a, Py_ssize_t n) {
    (void)self;
    return call_gemm(mkp_gemm, "gemm", a, n);
}
static PyObject* py_gemm_bt(PyObject* self, PyObject* const* a, Py_ssize_t n) {
    (void)self;
    return call_gemm(mkp_gemm_bt, "gemm_bt", a, n);
}
static PyObject* py_gemm_batched(PyObject* self, PyObject* const* a, Py_ssize_t n) {
    (void)self;
    return call_batched(mkp_gemm_batched, "gemm_batched", a, n);
}
static PyObject* py_gemm_batched_bt(PyObject* self, PyObject* const* a, Py_ssize_t n) {
    (void)self;
    return call_batched(mkp_gemm_batched_bt, "gemm_batched_bt", a, n);
}

static PyMethodDef methods[] = {
    {"gemm", (PyCFunction)(void (*)(void))py_gemm, METH_FASTCALL, "mkp_gemm"},
    {"gemm_bt", (PyCFunction)(void (*)(void))py_gemm_bt, METH_FASTCALL, "mkp_gemm_bt"},
    {"gemm_batched", (PyCFunction)(void (*)(void))py_gemm_batched, METH_FASTCALL, "mkp_gemm_batched"},
    {"gemm_batched_bt", (PyCFunction)(void (*)(void))py_gemm_batched_bt, METH_FASTCALL, "mkp_gemm_batched_bt"},
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_mkpfast", NULL, -1, methods, NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__mkpfast(void) { return PyModule_Create(&module); }
