"""Placeholder, replaced by the ctypes binding."""
__all__ = []
